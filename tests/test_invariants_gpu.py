"""Invariants of the scan checked on the GPU through the C ABI.

- pack order: every (sample, head) is its own recurrence with the state reset at the sample's
  first token (paper, Sec. 3 KDA paragraph), so permuting the samples of a pack permutes the
  per-sample results and changes none of them;
- value-column separability: the update S_t = (I - b k k^T) Diag(a) S_{t-1} + b k v^T acts on
  the columns of S one by one (explainer page, "One stream, three mechanisms, no positions"),
  so permuting or zeroing columns of V permutes or zeroes the same columns of O and S;
- the same results with every kernel launch serialised (AMD_SERIALIZE_KERNEL=3);
- KDA_VALIDATE=1 turns malformed sample tables into KDA_E_SEQLENS before any launch;
- KDA_DEBUG_SYNC=1 (each call waits for its stream) changes no result, and a call captured
  into a graph under it does not wait;
- kda_release gives the pooled workspace memory back to the driver.
"""
import json
import os
import subprocess
import sys
import tempfile

import numpy as np
import pytest

import gpu_util as gu
from delta_rule_recurrent_kda_amd import inputs

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from delta_rule_recurrent_kda_amd import kda
    kda.library()


def _bits(t):
    import torch
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t


def _repack(a, lens, order):
    """The pack with its samples in `order` (a list of sample indices)."""
    cu = np.concatenate([[0], np.cumsum(lens)])
    b = {}
    for x in ("q", "k", "v", "log_alpha", "beta"):
        b[x] = np.ascontiguousarray(np.concatenate([a[x][cu[n]:cu[n + 1]] for n in order]))
    b["cu_seqlens"] = np.concatenate([[0], np.cumsum([lens[n] for n in order])]).astype(np.int32)
    return b


# (name, sample lengths, heads): a pack that runs one chain per (sample, head) and one whose few
# long samples are cut into segments
PACKS = [("many", (700, 0, 1300, 65, 250, 31), 4), ("long_split", (5100, 2300, 130), 1)]


@pytest.mark.parametrize("name,lens,H", PACKS, ids=[p[0] for p in PACKS])
def test_pack_order_permutation(name, lens, H):
    import torch
    from delta_rule_recurrent_kda_amd import kda
    gu.log(f"case pack order {name}: lengths {lens}, {H} heads")
    spec = inputs.KdaSpec(f"perm_{name}", lens, H, 128, 128, "bf16", (0.0005, 0.05), 8181)
    a = inputs.generate(spec)
    order = list(np.random.default_rng(82).permutation(len(lens)))
    b = _repack(a, lens, order)
    res = []
    for pk in (a, b):
        d = gu.device_inputs(spec, pk)
        o, fs = kda.forward(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["cu_seqlens"])
        torch.cuda.synchronize()
        res.append((_bits(o).cpu().numpy(), fs.cpu().numpy()))
    (o1, f1), (o2, f2) = res
    cu1 = spec.cu_seqlens()
    cu2 = b["cu_seqlens"]
    for j, n in enumerate(order):
        assert np.array_equal(o1[cu1[n]:cu1[n + 1]], o2[cu2[j]:cu2[j + 1]]), (name, n)
        assert np.array_equal(f1[n], f2[j]), (name, n)
    # and the first pack against the oracle
    o_ref, f_ref = gu.oracle_ref(spec, a)
    out = o1.view(np.uint16).astype(np.uint32) << 16
    gu.compare(spec, out.view(np.float32).astype(np.float64), f1.astype(np.float64), o_ref, f_ref,
               label=f"pack order {name}")


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_value_columns_separate(dt):
    import torch
    from delta_rule_recurrent_kda_amd import kda
    gu.log(f"case value-column separability {dt}")
    spec = inputs.KdaSpec(f"cols_{dt}", (300, 0, 129, 2500), 2, 128, 128, dt, (0.001, 0.1), 8282)
    a = inputs.generate(spec)
    d = gu.device_inputs(spec, a)
    args = lambda v: (d["q"], d["k"], v, d["log_alpha"], d["beta"], d["cu_seqlens"])
    o, fs = kda.forward(*args(d["v"]))
    perm = torch.from_numpy(np.random.default_rng(83).permutation(spec.dv)).to("cuda:0")
    op, fsp = kda.forward(*args(d["v"][:, :, perm].contiguous()))
    zcols = torch.tensor([0, 5, 64, 127], device="cuda:0")
    vz = d["v"].clone()
    vz[:, :, zcols] = 0
    oz, fsz = kda.forward(*args(vz))
    torch.cuda.synchronize()
    assert torch.equal(_bits(op), _bits(o[:, :, perm].contiguous()))
    assert torch.equal(fsp, fs[..., perm].contiguous())
    assert torch.count_nonzero(oz[:, :, zcols].float()).item() == 0
    assert torch.count_nonzero(fsz[..., zcols]).item() == 0
    keep = torch.tensor([c for c in range(spec.dv) if c not in zcols.tolist()], device="cuda:0")
    assert torch.equal(_bits(oz[:, :, keep].contiguous()), _bits(o[:, :, keep].contiguous()))
    assert torch.equal(fsz[..., keep], fs[..., keep])


_SERIAL_CHILD = r"""
import json, sys
import numpy as np
import torch
sys.path.insert(0, sys.argv[1])
from delta_rule_recurrent_kda_amd import inputs, kda
spec = inputs.KdaSpec("serial", (700, 3000, 65), 2, 128, 128, "bf16", (0.001, 0.1), 8383)
a = inputs.generate(spec)
dev = "cuda:0"
t = {n: torch.from_numpy(a[n].view(np.int16)).view(torch.bfloat16).to(dev) for n in ("q", "k", "v", "log_alpha", "beta")}
cu = torch.from_numpy(a["cu_seqlens"]).to(dev)
o, fs = kda.forward(t["q"], t["k"], t["v"], t["log_alpha"], t["beta"], cu)
do = torch.ones_like(o)
g = kda.backward(t["q"], t["k"], t["v"], t["log_alpha"], t["beta"], cu, do)
torch.cuda.synchronize()
res = [o, fs] + [x for x in g if x is not None]
np.savez(sys.argv[2], *[(x.view(torch.int16) if x.dtype == torch.bfloat16 else x).cpu().numpy() for x in res])
print("child done", flush=True)
"""


def test_same_results_with_serialised_kernels(tmp_path):
    """A child process with AMD_SERIALIZE_KERNEL=3 (every launch waits for the previous one and
    is waited for) computes the forward and backward of the same inputs; results must equal
    this process's bit for bit."""
    gu.log("case serialised kernels (child process with AMD_SERIALIZE_KERNEL=3)")
    path = str(tmp_path / "serial.npz")
    env = dict(os.environ, AMD_SERIALIZE_KERNEL="3")
    r = subprocess.run([sys.executable, "-c", _SERIAL_CHILD, ROOT, path], env=env, capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    serial = np.load(path)
    here = str(tmp_path / "here.npz")
    r = subprocess.run([sys.executable, "-c", _SERIAL_CHILD, ROOT, here], capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    plain = np.load(here)
    assert len(serial.files) == len(plain.files) == 8
    for f in serial.files:
        assert np.array_equal(serial[f], plain[f]), f


def _bad_tables():
    # (cu_seqlens for T = 300, what is wrong)
    return [([0, 200, 100, 300], "decreasing"), ([5, 100, 200, 300], "first offset not 0"),
            ([0, 100, 200, 299], "last offset not T")]


@pytest.mark.parametrize("case", range(3))
def test_validate_rejects_malformed_offsets(monkeypatch, case):
    import torch
    from delta_rule_recurrent_kda_amd import kda
    cu_list, what = _bad_tables()[case]
    gu.log(f"case KDA_VALIDATE: {what}")
    monkeypatch.setenv("KDA_VALIDATE", "1")
    dev = "cuda:0"
    T, H, D = 300, 2, 128
    x = torch.zeros((T, H, D), dtype=torch.bfloat16, device=dev)
    beta = torch.zeros((T, H), dtype=torch.bfloat16, device=dev)
    cu = torch.tensor(cu_list, dtype=torch.int32, device=dev)
    out = torch.full((T, H, D), 7.0, dtype=torch.bfloat16, device=dev)
    with pytest.raises(kda.KdaError) as e:
        kda.kda_forward(x, x, x, x, beta, cu, out, None)
    assert e.value.status == 6, str(e.value)
    with pytest.raises(kda.KdaError) as e:
        kda.backward(x, x, x, x, beta, cu, torch.zeros_like(x))
    assert e.value.status == 6, str(e.value)
    torch.cuda.synchronize()
    assert torch.all(out.float() == 7.0)           # nothing was launched
    # the same offsets pass when they are well formed
    kda.kda_forward(x, x, x, x, beta, torch.tensor([0, 100, 200, 300], dtype=torch.int32, device=dev), out, None)
    torch.cuda.synchronize()


def test_validate_rejects_short_conv_grid_mismatch(monkeypatch):
    import torch
    from delta_rule_recurrent_kda_amd import kda
    gu.log("case KDA_VALIDATE: short convolution grid that does not match the sample")
    monkeypatch.setenv("KDA_VALIDATE", "1")
    dev = "cuda:0"
    x = torch.zeros((40, 16), dtype=torch.bfloat16, device=dev)
    wt = torch.zeros((4, 16), device=dev)
    wv = torch.zeros((3, 3, 3, 16), device=dev)
    cu = torch.tensor([0, 40], dtype=torch.int32, device=dev)
    tl = torch.tensor([4], dtype=torch.int32, device=dev)
    with pytest.raises(kda.KdaError) as e:
        kda.short_conv(x, wt, wv, cu, tl, torch.tensor([[2, 3, 5]], dtype=torch.int32, device=dev))
    assert e.value.status == 6
    kda.short_conv(x, wt, wv, cu, tl, torch.tensor([[2, 3, 6]], dtype=torch.int32, device=dev))
    torch.cuda.synchronize()


def test_release_returns_pool_memory():
    """After a backward whose workspace is several hundred MB, the freed workspace stays in the
    device's pool (free device memory does not come back); kda_release gives it to the driver."""
    import torch
    from delta_rule_recurrent_kda_amd import kda
    gu.log("case kda_release returns memory")
    dev = "cuda:0"
    T, H, D = 16384, 4, 128
    g = torch.Generator(device=dev)
    g.manual_seed(84)
    q = torch.nn.functional.normalize(torch.randn((T, H, D), device=dev, generator=g), dim=-1).to(torch.bfloat16)
    v = torch.randn((T, H, D), device=dev, generator=g).to(torch.bfloat16)
    la = torch.full((T, H, D), -0.01, device=dev).to(torch.bfloat16)
    beta = torch.full((T, H), 0.5, device=dev).to(torch.bfloat16)
    cu = torch.tensor([0, 5000, T], dtype=torch.int32, device=dev)
    do = torch.ones_like(v)
    ws = kda.backward_workspace_bytes(T, 2, H, D, D)
    assert ws > 200 << 20
    kda.backward(q, q, v, la, beta, cu, do)
    torch.cuda.synchronize()
    free0, _ = torch.cuda.mem_get_info()
    kda.release()
    torch.cuda.synchronize()
    free1, _ = torch.cuda.mem_get_info()
    gu.log(f"[release] workspace {ws / 2**20:.0f} MiB, free memory +{(free1 - free0) / 2**20:.0f} MiB")
    assert free1 - free0 >= ws // 2, (free0, free1, ws)


def test_debug_sync_same_results(monkeypatch):
    """Forward, backward and short convolution with KDA_DEBUG_SYNC=1 return KDA_OK and the same
    results bit for bit; under stream capture the call does not synchronise (which capture
    forbids), and the replayed graph gives the eager result."""
    import torch
    from delta_rule_recurrent_kda_amd import kda
    gu.log("case KDA_DEBUG_SYNC")
    spec = inputs.custom([700, 0, 1300, 65], heads=2, d=128, seed=33)
    d = gu.device_inputs(spec, inputs.generate(spec))
    dev = "cuda:0"
    T, H, N = spec.total_tokens, spec.heads, len(spec.seq_lens)
    g = torch.Generator(device=dev)
    g.manual_seed(35)
    do = torch.randn((T, H, spec.dv), device=dev, generator=g).to(torch.bfloat16)
    x = torch.randn((90, 32), device=dev, generator=g).to(torch.bfloat16)
    wt = torch.randn((4, 32), device=dev, generator=g)
    wv = torch.randn((3, 3, 3, 32), device=dev, generator=g)
    ccu = torch.tensor([0, 40, 90], dtype=torch.int32, device=dev)
    tl = torch.tensor([4, 2], dtype=torch.int32, device=dev)
    grid = torch.tensor([[2, 3, 6], [2, 4, 6]], dtype=torch.int32, device=dev)

    def run_all():
        o = kda.forward(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["cu_seqlens"])
        gr = kda.backward(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["cu_seqlens"], do)
        y = kda.short_conv(x, wt, wv, ccu, tl, grid)
        torch.cuda.synchronize()
        return [t.clone() for t in (list(o) + list(gr) + [y])]

    plain = run_all()
    monkeypatch.setenv("KDA_DEBUG_SYNC", "1")
    synced = run_all()
    assert len(plain) == len(synced)
    for i, (a, b) in enumerate(zip(plain, synced)):
        assert torch.equal(_bits(a), _bits(b)), i
    # captured: the forward records its kernels and no wait
    out = torch.empty((T, H, spec.dv), dtype=torch.bfloat16, device=dev)
    fs = torch.empty((N, H, spec.dk, spec.dv), dtype=torch.float32, device=dev)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        kda.kda_forward(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["cu_seqlens"], out, fs,
                        stream=torch.cuda.current_stream())
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        kda.kda_forward(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["cu_seqlens"], out, fs,
                        stream=torch.cuda.current_stream())
    out.zero_()
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    assert torch.equal(_bits(out), _bits(plain[0]))
    assert torch.equal(fs, plain[1])
