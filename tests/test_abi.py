"""C ABI: the library loads, exports what include/kda.h declares, and rejects
bad arguments before touching the device (CPU only: no launches here)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")


@pytest.fixture(scope="module")
def lib():
    from delta_rule_recurrent_kda_amd import build as kbuild
    from delta_rule_recurrent_kda_amd import kda
    if kbuild.is_stale():
        kbuild.build()
    return kda.library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_boundary():
    assert {"kda_forward", "kda_forward_from_state", "kda_forward_ex", "kda_backward", "kda_backward_workspace_bytes",
            "kda_short_conv", "kda_short_conv_backward", "kda_workspace_bytes", "kda_timing_enable",
            "kda_timing_read", "kda_release", "kda_status_str", "kda_last_error", "kda_version"} <= set(declared_functions())


def test_release_before_any_call_is_ok(lib):
    assert lib.kda_release() == 0


def test_every_declared_symbol_is_exported(lib):
    from delta_rule_recurrent_kda_amd import kda
    nm = subprocess.run(["nm", "-D", "--defined-only", kda.LIB_PATH], capture_output=True, text=True,
                        check=True).stdout
    exported = set(re.findall(r"\bT (kda_\w+)$", nm, flags=re.M))
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(lib, name)


def test_header_compiles_as_c(tmp_path):
    src = tmp_path / "t.c"
    src.write_text('#include "kda.h"\nint main(void){ return (int)kda_version() < 0; }\n')
    subprocess.run(["gcc", "-std=c11", "-fsyntax-only", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
                    "-I", "/opt/rocm/include", str(src)], check=True)


def test_status_strings(lib):
    assert lib.kda_status_str(0) == b"KDA_OK"
    assert lib.kda_status_str(5) == b"KDA_E_UNSUPPORTED"
    assert lib.kda_version() >= 100


def _call(kw):
    from delta_rule_recurrent_kda_amd import kda
    a = dict(q=0x100000, k=0x200000, v=0x300000, log_alpha=0x400000, beta=0x500000, cu_seqlens=0x600000,
             out=0x700000, final_state=0x800000, total_tokens=128, num_seqs=1, num_heads=2, d_k=128,
             d_v=128, dtype=kda.KDA_BF16, stream=None)
    a.update(kw)
    st = kda.kda_forward_raw(**a)
    return st, kda.library().kda_last_error().decode()


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=7), 2),
    (dict(total_tokens=-1), 3),
    (dict(num_heads=0), 3),
    (dict(num_seqs=-2), 3),
    (dict(d_k=96), 5),
    (dict(d_v=256), 5),
    (dict(cu_seqlens=None), 1),
    (dict(q=None), 1),
    (dict(out=None), 1),
    (dict(v=0x300008), 4),
    (dict(final_state=0x800004), 4),
    (dict(out=0x100000), 3),
    (dict(out=0x108000), 3),                           # out starts inside q
    (dict(final_state=0x708000), 3),                   # final_state overlaps out
    (dict(total_tokens=1 << 26, num_heads=64), 5),
])
def test_bad_arguments_are_rejected_without_launch(lib, kw, code):
    st, msg = _call(kw)
    assert st == code, (st, msg)
    assert msg


def test_empty_batch_is_a_no_op(lib):
    st, _ = _call(dict(num_seqs=0, total_tokens=0))
    assert st == 0


def _call_from_state(kw):
    from delta_rule_recurrent_kda_amd import kda
    a = dict(q=0x100000, k=0x200000, v=0x300000, log_alpha=0x400000, beta=0x500000, cu_seqlens=0x600000,
             initial_state=0x900000, out=0x700000, final_state=0x800000, total_tokens=128, num_seqs=1,
             num_heads=2, d_k=128, d_v=128, dtype=kda.KDA_BF16, stream=None)
    a.update(kw)
    st = kda.kda_forward_from_state_raw(**a)
    return st, kda.library().kda_last_error().decode()


@pytest.mark.parametrize("kw,code", [
    (dict(initial_state=0x900004), 4),                 # misaligned
    (dict(final_state=0x900000), 3),                   # final_state aliases initial_state
    (dict(d_k=96), 5),
    (dict(q=None), 1),
])
def test_from_state_bad_arguments_are_rejected_without_launch(lib, kw, code):
    st, msg = _call_from_state(kw)
    assert st == code, (st, msg)
    assert msg


def _call_ex(kw):
    from delta_rule_recurrent_kda_amd import kda
    a = dict(q=0x100000, k=0x200000, v=0x300000, log_alpha=0x400000, beta=0x500000, cu_seqlens=0x600000,
             initial_state=None, out=0x700000, final_state=0x800000, total_tokens=128, num_seqs=1,
             num_heads=2, d_k=128, d_v=128, dtype=kda.KDA_BF16, options=kda.KDA_OPT_QK_L2NORM,
             stream=None)
    a.update(kw)
    st = kda.kda_forward_ex_raw(**a)
    return st, kda.library().kda_last_error().decode()


@pytest.mark.parametrize("kw,code", [
    (dict(options=2), 5),                            # unknown option bit
    (dict(options=0x80000001), 5),
    (dict(d_v=96), 5),
    (dict(k=None), 1),
    (dict(out=0x200000), 3),
])
def test_forward_ex_bad_arguments_are_rejected_without_launch(lib, kw, code):
    st, msg = _call_ex(kw)
    assert st == code, (st, msg)
    assert msg


def test_forward_ex_empty_batch_is_a_no_op(lib):
    st, _ = _call_ex(dict(num_seqs=0, total_tokens=0))
    assert st == 0


def _call_noalloc(kw):
    from delta_rule_recurrent_kda_amd import kda
    a = dict(q=0x100000, k=0x200000, v=0x300000, log_alpha=0x400000, beta=0x500000, cu_seqlens=0x600000,
             initial_state=None, out=0x700000, final_state=0x800000, total_tokens=128, num_seqs=1,
             num_heads=2, d_k=128, d_v=128, dtype=kda.KDA_BF16, options=0, stream=None)
    a.update(kw)
    st = kda.kda_forward_noalloc_raw(**a)
    return st, kda.library().kda_last_error().decode()


@pytest.mark.parametrize("kw,code", [
    (dict(options=2), 5),
    (dict(d_k=96), 5),
    (dict(beta=None), 1),
    (dict(v=0x300008), 4),
    (dict(final_state=0x100000), 3),                 # final_state aliases q
    (dict(dtype=7), 2),
])
def test_forward_noalloc_bad_arguments_are_rejected_without_launch(lib, kw, code):
    st, msg = _call_noalloc(kw)
    assert st == code, (st, msg)
    assert msg


def test_forward_noalloc_empty_batch_is_a_no_op(lib):
    st, _ = _call_noalloc(dict(num_seqs=0, total_tokens=0))
    assert st == 0


def _call_conv(kw):
    from delta_rule_recurrent_kda_amd import kda
    a = dict(x=0x100000, w_text=0x200000, w_vis=0x300000, cu_seqlens=0x400000, text_len=0x500000, grid=0x600000,
             y=0x700000, total_tokens=100, num_seqs=1, channels=64, k_text=4, k_t=3, k_h=3, k_w=3,
             dtype=kda.KDA_BF16, stream=None)
    a.update(kw)
    st = kda.short_conv_raw(**a)
    return st, kda.library().kda_last_error().decode()


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=3), 2),
    (dict(channels=60), 5),
    (dict(k_text=9), 5),
    (dict(k_t=5), 5),
    (dict(k_h=2), 5),
    (dict(k_w=7), 5),
    (dict(total_tokens=-1), 3),
    (dict(grid=None), 1),
    (dict(x=None), 1),
    (dict(y=0x700008), 4),
    (dict(y=0x100000), 3),
    (dict(y=0x100800), 3),                             # y starts inside x
    (dict(y=0x5fff00), 3),                             # y runs into grid
    (dict(total_tokens=1 << 25), 5),
])
def test_short_conv_bad_arguments_are_rejected_without_launch(lib, kw, code):
    st, msg = _call_conv(kw)
    assert st == code, (st, msg)
    assert msg


def test_short_conv_with_no_samples_takes_null_tables(lib):
    st, msg = _call_conv(dict(num_seqs=0, total_tokens=0, text_len=None, grid=None))
    assert st == 0, msg


def _call_conv_bwd(kw):
    from delta_rule_recurrent_kda_amd import kda
    a = dict(x=0x100000, w_text=0x200000, w_vis=0x300000, cu_seqlens=0x400000, text_len=0x500000, grid=0x600000,
             dy=0x700000, dx=0x800000, dw_text=0x900000, dw_vis=0xa00000, total_tokens=100, num_seqs=1,
             channels=64, k_text=4, k_t=3, k_h=3, k_w=3, dtype=kda.KDA_BF16, stream=None)
    a.update(kw)
    st = kda.short_conv_backward_raw(**a)
    return st, kda.library().kda_last_error().decode()


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=3), 2),
    (dict(channels=12), 5),
    (dict(k_w=4), 5),
    (dict(k_t=0), 5),
    (dict(dy=None), 1),
    (dict(dx=None), 1),
    (dict(dw_vis=None), 1),
    (dict(dy=0x700004), 4),
    (dict(dx=0x800008), 4),
    (dict(dx=0x700000), 3),                            # dx aliases dy
    (dict(dw_text=0x100040), 3),                       # dw_text starts inside x
    (dict(dw_vis=0x8ffff0), 3),                        # dw_vis runs into dw_text
    (dict(dw_text=0x300100), 3),                       # dw_text inside w_vis
    (dict(total_tokens=1 << 25), 5),
])
def test_short_conv_backward_bad_arguments_are_rejected_without_launch(lib, kw, code):
    st, msg = _call_conv_bwd(kw)
    assert st == code, (st, msg)
    assert msg


def _call_bwd(kw):
    from delta_rule_recurrent_kda_amd import kda
    a = dict(q=0x100000, k=0x200000, v=0x300000, log_alpha=0x400000, beta=0x500000, cu_seqlens=0x600000,
             initial_state=None, d_out=0x700000, d_final_state=None, dq=0x800000, dk=0x900000, dv=0xa00000,
             dlog_alpha=0xb00000, dbeta=0xc00000, d_initial_state=None, total_tokens=128, num_seqs=1,
             num_heads=2, d_k=128, d_v=128, dtype=kda.KDA_BF16, options=0, stream=None)
    a.update(kw)
    st = kda.kda_backward_raw(**a)
    return st, kda.library().kda_last_error().decode()


@pytest.mark.parametrize("kw,code", [
    (dict(options=4), 5),
    (dict(dtype=9), 2),
    (dict(d_k=32), 5),
    (dict(d_out=None), 1),
    (dict(dbeta=None), 1),
    (dict(dv=0xa00008), 4),
    (dict(dq=0x100000), 3),                            # a gradient aliases an input
    (dict(dk=0x800000), 3),                            # two gradients alias
    (dict(d_initial_state=0x600000), 3),
    (dict(dk=0x808000), 3),                            # dk starts inside dq
    (dict(dbeta=0x5ffff0), 3),                         # dbeta runs into cu_seqlens
])
def test_backward_bad_arguments_are_rejected_without_launch(lib, kw, code):
    st, msg = _call_bwd(kw)
    assert st == code, (st, msg)
    assert msg


def test_backward_workspace_bytes(lib):
    from delta_rule_recurrent_kda_amd import kda
    # 32-token chunks: chunk table, one fp32 record (Kh, Kc, Qh [32][d_k], T, P, M [32][32], gamma,
    # b, 1/|q|, 1/|k|) and the state and its gradient (fp32 [d_k][d_v] each) per (chunk, head)
    T, N, H = 1000, 3, 2
    chunks = (T + 31) // 32 + N
    rec = (3 * 32 * 128 + 3 * 32 * 32 + 128 + 3 * 32) * 4
    table = ((3 * N + 2) * 4 + 255) // 256 * 256      # chunk and segment tables, longest-first order
    assert kda.backward_workspace_bytes(T, N, H, 128, 128) == table + chunks * H * (rec + 2 * 128 * 128 * 4)
    assert kda.backward_workspace_bytes(T, 0, H, 128, 128) == 0


def test_workspace_bytes(lib, monkeypatch):
    from delta_rule_recurrent_kda_amd import kda
    rec = {(128, 128): 74240, (128, 64): 74240 - 8192}
    # record: -W, Qh (4*d_k/32 fragments of 1 KB each), Kb^T (d_k/16 * 2 KB), P (8 KB),
    # gamma (4 d_k bytes), U (d_v/16 * 2 KB); plus the chunk table rounded up to 256 bytes
    def record(dk, dv):
        return 2 * (4 * dk // 32 * 512) * 2 + (dk // 16) * 2 * 1024 + 8192 + 4 * dk + (dv // 16) * 2048
    assert record(128, 128) == rec[(128, 128)] and record(128, 64) == rec[(128, 64)]
    # chunk and segment offset tables (rounded up to 256 bytes), one record per
    # (64-token chunk, head) for the upper bound ceil(T / 64) + N of chunks, and, when the
    # chain would get at most 64 workgroups, per-segment local states and transitions (fp32)
    cases = [(17108, 8, 16, 128, 128), (1, 1, 1, 64, 64), (189272, 1, 16, 128, 64), (640, 300, 3, 64, 128),
             (189272, 1, 16, 128, 128), (5000, 1, 2, 128, 128), (100000, 100, 2, 128, 128), (4000, 600, 1, 128, 128)]
    for fused, T, N, H, dk, dv in [(False,) + c for c in cases] + [(True,) + c for c in cases]:
        if fused:
            monkeypatch.delenv("KDA_SCAN_VARIANT", raising=False)     # the default
        else:
            monkeypatch.setenv("KDA_SCAN_VARIANT", "wy")
        if dk == 128 and dv == 128 and fused:
            # fused scan (32-token chunks): 256 bytes of unit counters; when the (sample, head)
            # units are fewer than 256, segments of lseg chunks, each (segment, head) with an fp32
            # local state and its transition (64 KB each), and a segment table for more than 64 samples
            chunks = (T + 31) // 32 + N
            expect = 256
            if N * H < 256:
                lseg = max(16, (chunks * H + 255) // 256)
                if lseg < chunks:
                    max_segs = (chunks + lseg - 1) // lseg + N
                    expect += max_segs * H * 2 * 65536 + ((N + 1) * 4 + 255) // 256 * 256 * (N > 64)
            assert kda.workspace_bytes(T, N, H, dk, dv, kda.KDA_BF16) == expect, (T, N, H, dk, dv)
            continue
        bound = (T + 63) // 64
        chunks = bound + N
        table = (2 * (N + 1) * 4 + 255) // 256 * 256
        expect = table + chunks * H * record(dk, dv)
        if N * H * (dv // 64) <= 64:
            segs = max(1, 256 // (H * (dv // 64)))
            lseg = max(32, (bound + segs - 1) // segs)
            if lseg < bound:
                max_segs = (bound + N + lseg - 1) // lseg + N
                expect += max_segs * H * dk * (dv + dk) * 4
        assert kda.workspace_bytes(T, N, H, dk, dv, kda.KDA_BF16) == expect, (T, N, H, dk, dv)
    assert kda.workspace_bytes(1000, 2, 2, 128, 128, kda.KDA_F32) == 0
    assert kda.workspace_bytes(1000, 0, 2, 128, 128, kda.KDA_BF16) == 0
    assert kda.workspace_bytes(1000, 2, 2, 96, 128, kda.KDA_BF16) == 0
    monkeypatch.setenv("KDA_SCAN_VARIANT", "sequential")
    assert kda.workspace_bytes(17108, 8, 16, 128, 128, kda.KDA_BF16) == 0


def test_bandwidth_probe_library_builds_and_exports(lib):
    from delta_rule_recurrent_kda_amd import build as kbuild
    assert os.path.exists(kbuild.PROBE_LIB)
    nm = subprocess.run(["nm", "-D", "--defined-only", kbuild.PROBE_LIB], capture_output=True, text=True,
                        check=True).stdout
    assert re.search(r"\bT kda_bw_probe$", nm, flags=re.M)
    probe = ctypes.CDLL(kbuild.PROBE_LIB)
    probe.kda_bw_probe.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int,
                                   ctypes.c_void_p]
    # bad arguments are refused before any launch
    assert probe.kda_bw_probe(0, None, None, 16, 1, None) != 0
    assert probe.kda_bw_probe(2, 0x100000, 0x200000, 16, 1, None) != 0
    assert probe.kda_bw_probe(0, 0x100000, 0x200000, 15, 1, None) != 0
