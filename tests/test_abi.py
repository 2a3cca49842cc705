"""The C ABI library loads and exports what include/wkv6.h declares; argument
checks that return before any GPU work behave as documented.  No compute
call is made here, so this runs without a GPU (it needs the built library,
which __graft_entry__.build() or `python -m linear_attention_rnn_amd.build`
produces)."""
import ctypes
import os

import pytest

from linear_attention_rnn_amd import wkv6

pytestmark = pytest.mark.skipif(not os.path.exists(wkv6.LIB_PATH),
                                reason="libwkv6.so not built")

A = 0x10000  # fake, 16-byte aligned addresses: never dereferenced by these calls


def test_exports_every_declared_function():
    names = wkv6.header_functions()
    assert set(names) == {"wkv6_fwd", "wkv6_fwd_noalloc", "wkv6_group_norm_gate", "wkv6_fwd_workspace_bytes", "wkv6_workspace_reserved_bytes", "wkv6_trim_workspace", "wkv6_fwd_gn", "wkv5_fwd", "wkv4_fwd", "wkv6_fwd_state", "wkv6_bwd", "wkv6_status_str",
                          "wkv6_last_error", "wkv6_abi_version"}
    L = wkv6.lib()
    for n in names:
        assert hasattr(L, n), f"{n} not exported"
        assert ctypes.cast(getattr(L, n), ctypes.c_void_p).value


def test_abi_version_and_status_strings():
    assert wkv6.abi_version() == 7
    assert wkv6.status_str(0) == "ok"
    texts = {wkv6.status_str(s) for s in range(5)}
    assert len(texts) == 5
    assert wkv6.status_str(99) == "unknown status"


def _call(B=2, T=8, C=128, H=2, ptrs=None, mode=0, dtype=0):
    p = ptrs or [A, A + 0x100000, A + 0x200000, A + 0x300000, A + 0x400000, A + 0x500000]
    return wkv6.fwd_raw(B, T, C, H, *p, mode, dtype, 0)


@pytest.mark.parametrize("kw,status", [
    (dict(B=-1), wkv6.ERR_INVALID_ARG),
    (dict(T=-3), wkv6.ERR_INVALID_ARG),
    (dict(C=-64), wkv6.ERR_INVALID_ARG),
    (dict(H=0), wkv6.ERR_INVALID_ARG),
    (dict(C=130, H=4), wkv6.ERR_INVALID_ARG),     # C not a multiple of H
    (dict(mode=2), wkv6.ERR_INVALID_ARG),
    (dict(dtype=5), wkv6.ERR_INVALID_ARG),
    (dict(C=96, H=2), wkv6.ERR_UNSUPPORTED),      # head size 48
    (dict(C=256, H=2), wkv6.ERR_UNSUPPORTED),     # head size 128
    (dict(T=2 ** 31), wkv6.ERR_UNSUPPORTED),
    (dict(T=2 ** 20, C=512, H=8), wkv6.ERR_UNSUPPORTED),   # one slice beyond 2 GiB of fp32 rows
    (dict(B=2 ** 24, T=1, C=64, H=1), wkv6.ERR_UNSUPPORTED),   # B * H * 256 work-items reach 2^32
    (dict(B=2 ** 12, T=1, C=64 * 2 ** 12, H=2 ** 12), wkv6.ERR_UNSUPPORTED),
    (dict(B=2 ** 62, T=1, C=64 * 2 ** 10, H=2 ** 10), wkv6.ERR_UNSUPPORTED),   # B * H overflows int64
])
def test_rejects_bad_arguments(kw, status):
    assert _call(**kw) == status
    assert wkv6.last_error() != ""


def test_last_error_is_per_thread():
    """Two host threads fail in different ways at the same time; each then
    reads the detail of its own call (the library's one piece of state is
    kept per thread)."""
    import threading

    both_failed = threading.Barrier(2)
    seen = {}

    def worker(name, kw):
        status = _call(**kw)
        both_failed.wait()   # neither reads its message before both calls have failed
        seen[name] = (status, wkv6.last_error())

    threads = [threading.Thread(target=worker, args=("mode", dict(mode=2))),
               threading.Thread(target=worker, args=("head", dict(C=96, H=2)))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=30)
    assert seen["mode"][0] == wkv6.ERR_INVALID_ARG and "mode" in seen["mode"][1]
    assert seen["head"][0] == wkv6.ERR_UNSUPPORTED and "head size" in seen["head"][1]


def test_empty_problem_is_a_noop():
    assert _call(B=0, ptrs=[0] * 6) == wkv6.OK
    assert _call(T=0, ptrs=[0] * 6) == wkv6.OK
    assert wkv6.last_error() == ""


@pytest.mark.parametrize("which", range(6))
def test_null_pointer(which):
    p = [A + 0x100000 * i for i in range(6)]
    p[which] = 0
    assert _call(ptrs=p) == wkv6.ERR_INVALID_ARG
    assert "null" in wkv6.last_error()


@pytest.mark.parametrize("which", range(6))
def test_misaligned_pointer(which):
    p = [A + 0x100000 * i for i in range(6)]
    p[which] += 4
    assert _call(ptrs=p) == wkv6.ERR_MISALIGNED


@pytest.mark.parametrize("which", range(5))
def test_output_overlapping_an_input(which):
    p = [A + 0x100000 * i for i in range(6)]
    p[5] = p[which] + 16
    assert _call(ptrs=p) == wkv6.ERR_INVALID_ARG
    assert "overlaps" in wkv6.last_error()


# ---- wkv6_fwd_state: the same checks plus the state buffers
S_IN, S_OUT = A + 0x600000, A + 0x700000


def _call_state(B=2, T=8, C=128, H=2, ptrs=None, s_in=S_IN, s_out=S_OUT, dtype=0):
    p = ptrs or [A, A + 0x100000, A + 0x200000, A + 0x300000, A + 0x400000, A + 0x500000]
    return wkv6.fwd_state_raw(B, T, C, H, *p, s_in, s_out, dtype, 0)


@pytest.mark.parametrize("kw,status", [
    (dict(B=-1), wkv6.ERR_INVALID_ARG),
    (dict(H=0), wkv6.ERR_INVALID_ARG),
    (dict(dtype=7), wkv6.ERR_INVALID_ARG),
    (dict(C=96, H=2), wkv6.ERR_UNSUPPORTED),
    (dict(s_in=S_IN + 8), wkv6.ERR_MISALIGNED),
    (dict(s_out=S_OUT + 4), wkv6.ERR_MISALIGNED),
    (dict(s_out=S_IN + 64), wkv6.ERR_INVALID_ARG),           # s_out overlaps s_in
    (dict(s_out=A + 0x500000 + 16), wkv6.ERR_INVALID_ARG),   # s_out overlaps y
    (dict(s_out=A + 0x100000), wkv6.ERR_INVALID_ARG),        # s_out overlaps k
    (dict(s_in=A + 0x500000 + 32), wkv6.ERR_INVALID_ARG),    # y overlaps s_in
    (dict(T=2 ** 31), wkv6.ERR_UNSUPPORTED),
])
def test_state_call_rejects_bad_arguments(kw, status):
    assert _call_state(**kw) == status
    assert wkv6.last_error() != ""


@pytest.mark.parametrize("which", range(6))
def test_state_call_null_tensor(which):
    p = [A + 0x100000 * i for i in range(6)]
    p[which] = 0
    assert _call_state(ptrs=p) == wkv6.ERR_INVALID_ARG


def test_state_call_empty_batch_is_a_noop():
    assert _call_state(B=0, ptrs=[0] * 6, s_in=0, s_out=0) == wkv6.OK
    assert _call_state(T=0, ptrs=[0] * 6, s_in=0, s_out=0) == wkv6.OK   # nothing to copy
    assert wkv6.last_error() == ""


# ---- wkv6_bwd: the same size checks; outputs clear of the inputs and of each other
def _call_bwd(B=2, T=8, C=128, H=2, ptrs=None, mode=0, dtype=0):
    p = ptrs or [A + 0x100000 * i for i in range(11)]
    return wkv6.bwd_raw(B, T, C, H, *p, mode, dtype, 0)


@pytest.mark.parametrize("kw,status", [
    (dict(B=-1), wkv6.ERR_INVALID_ARG),
    (dict(mode=3), wkv6.ERR_INVALID_ARG),
    (dict(C=96, H=2), wkv6.ERR_UNSUPPORTED),
    (dict(T=2 ** 31), wkv6.ERR_UNSUPPORTED),
])
def test_bwd_rejects_bad_sizes(kw, status):
    assert _call_bwd(**kw) == status


@pytest.mark.parametrize("which", range(11))
def test_bwd_null_pointer(which):
    p = [A + 0x100000 * i for i in range(11)]
    p[which] = 0
    assert _call_bwd(ptrs=p) == wkv6.ERR_INVALID_ARG


@pytest.mark.parametrize("which", range(11))
def test_bwd_misaligned_pointer(which):
    p = [A + 0x100000 * i for i in range(11)]
    p[which] += 8
    assert _call_bwd(ptrs=p) == wkv6.ERR_MISALIGNED


@pytest.mark.parametrize("out,other", [(6, 0), (7, 5), (8, 9), (9, 6), (10, 2), (6, 10)])
def test_bwd_overlapping_output(out, other):
    p = [A + 0x100000 * i for i in range(11)]
    p[out] = p[other] + 16
    assert _call_bwd(ptrs=p) == wkv6.ERR_INVALID_ARG
    assert "overlaps" in wkv6.last_error()


def test_bwd_empty_batch_is_a_noop():
    assert _call_bwd(B=0, ptrs=[0] * 11) == wkv6.OK


# ---- wkv5_fwd: wkv6_fwd's checks; w_raw holds only C values
def _call5(B=2, T=8, C=128, H=2, ptrs=None, mode=0, dtype=0):
    p = ptrs or [A, A + 0x100000, A + 0x200000, A + 0x300000, A + 0x400000, A + 0x500000]
    return wkv6.fwd5_raw(B, T, C, H, *p, mode, dtype, 0)


@pytest.mark.parametrize("kw,status", [
    (dict(B=-1), wkv6.ERR_INVALID_ARG),
    (dict(mode=2), wkv6.ERR_INVALID_ARG),
    (dict(C=96, H=2), wkv6.ERR_UNSUPPORTED),
    (dict(T=2 ** 31), wkv6.ERR_UNSUPPORTED),
])
def test_wkv5_rejects_bad_sizes(kw, status):
    assert _call5(**kw) == status


@pytest.mark.parametrize("which", range(6))
def test_wkv5_null_and_misaligned(which):
    p = [A + 0x100000 * i for i in range(6)]
    p[which] = 0
    assert _call5(ptrs=p) == wkv6.ERR_INVALID_ARG
    p[which] = A + 0x100000 * which + 4
    assert _call5(ptrs=p) == wkv6.ERR_MISALIGNED


def test_wkv5_output_overlap_counts_c_values_of_w():
    p = [A + 0x100000 * i for i in range(6)]
    p[5] = p[3] + 128 * 4 - 16          # y starts inside the 128 fp32 values of w_raw
    assert _call5(ptrs=p) == wkv6.ERR_INVALID_ARG
    assert "overlaps w_raw" in wkv6.last_error()


def test_wkv5_empty_problem_is_a_noop():
    assert _call5(B=0, ptrs=[0] * 6) == wkv6.OK
    assert _call5(T=0, ptrs=[0] * 6) == wkv6.OK


# ---- wkv4_fwd: per-channel operator, no heads
def _call4(B=2, T=8, C=100, ptrs=None, dtype=0):
    p = ptrs or [A + 0x100000 * i for i in range(5)]
    return wkv6.fwd4_raw(B, T, C, *p, dtype, 0)


@pytest.mark.parametrize("kw,status", [
    (dict(B=-1), wkv6.ERR_INVALID_ARG),
    (dict(T=-1), wkv6.ERR_INVALID_ARG),
    (dict(C=-5), wkv6.ERR_INVALID_ARG),
    (dict(dtype=3), wkv6.ERR_INVALID_ARG),
    (dict(C=256 * 65536), wkv6.ERR_UNSUPPORTED),      # more channel blocks than grid rows
    (dict(B=2 ** 31), wkv6.ERR_UNSUPPORTED),
])
def test_wkv4_rejects_bad_sizes(kw, status):
    assert _call4(**kw) == status


@pytest.mark.parametrize("which", range(5))
def test_wkv4_null_misaligned_overlap(which):
    p = [A + 0x100000 * i for i in range(5)]
    p[which] = 0
    assert _call4(ptrs=p) == wkv6.ERR_INVALID_ARG
    p[which] = A + 0x100000 * which + 8
    assert _call4(ptrs=p) == wkv6.ERR_MISALIGNED
    if which < 4:
        p = [A + 0x100000 * i for i in range(5)]
        p[4] = p[which] + 16
        assert _call4(ptrs=p) == wkv6.ERR_INVALID_ARG and "overlaps" in wkv6.last_error()


def test_wkv4_empty_problem_is_a_noop():
    for kw in (dict(B=0), dict(T=0), dict(C=0)):
        assert _call4(ptrs=[0] * 5, **kw) == wkv6.OK


# ---- wkv6_fwd_gn: wkv6_fwd's checks plus the gate, affine and eps
# pointers: r, k, v, w_raw, u, g, gamma, beta, out
def _call_gn(B=2, T=8, C=128, H=2, ptrs=None, eps=1e-5, mode=0, dtype=0):
    p = ptrs or [A + 0x100000 * i for i in range(9)]
    return wkv6.fwd_gn_raw(B, T, C, H, *p[:8], eps, p[8], mode, dtype, 0)


@pytest.mark.parametrize("kw,status", [
    (dict(B=-1), wkv6.ERR_INVALID_ARG),
    (dict(mode=4), wkv6.ERR_INVALID_ARG),
    (dict(C=96, H=2), wkv6.ERR_UNSUPPORTED),
    (dict(eps=-1.0), wkv6.ERR_INVALID_ARG),
    (dict(eps=float("nan")), wkv6.ERR_INVALID_ARG),
    (dict(eps=float("inf")), wkv6.ERR_INVALID_ARG),
])
def test_gn_rejects_bad_arguments(kw, status):
    assert _call_gn(**kw) == status


@pytest.mark.parametrize("which", range(9))
def test_gn_null_misaligned_overlap(which):
    p = [A + 0x100000 * i for i in range(9)]
    p[which] = 0
    assert _call_gn(ptrs=p) == wkv6.ERR_INVALID_ARG
    p[which] = A + 0x100000 * which + 4
    assert _call_gn(ptrs=p) == wkv6.ERR_MISALIGNED
    if which != 8:
        p = [A + 0x100000 * i for i in range(9)]
        p[8] = p[which] + 16
        assert _call_gn(ptrs=p) == wkv6.ERR_INVALID_ARG and "overlaps" in wkv6.last_error()


def test_gn_empty_problem_is_a_noop():
    assert _call_gn(B=0, ptrs=[0] * 9) == wkv6.OK
    assert _call_gn(T=0, ptrs=[0] * 9) == wkv6.OK


def test_fwd_workspace_bytes_follows_the_documented_formula():
    """wkv6_fwd_workspace_bytes (host arithmetic, no GPU): zero for calls that
    are not cut into segments (enough (batch, head) pairs, or at most four
    causal tokens), else B*H*segments*2*(64*64+64)*4 bytes, as include/wkv6.h
    documents, with 1 < segments <= the number of 64-token chunks."""
    per = 2 * (64 * 64 + 64) * 4
    assert wkv6.fwd_workspace_bytes(64, 196, 768, 12, "bidirectional") == 0   # image-base: 768 pairs
    assert wkv6.fwd_workspace_bytes(8, 4, 2048, 32, "causal") == 0            # decode kernel
    assert wkv6.fwd_workspace_bytes(-1, 4, 128, 2) == 0                       # invalid sizes
    for B, T, C, H, mode, bf16 in ((8, 4096, 2048, 32, "causal", True), (4, 4096, 1024, 16, "bidirectional", True),
                                   (1, 1000, 128, 2, "causal", False), (2, 587, 192, 3, "bidirectional", True)):
        n = wkv6.fwd_workspace_bytes(B, T, C, H, mode, bf16)
        assert n > 0 and n % (B * H * per) == 0, (B, T, n)
        G = n // (B * H * per)
        assert 1 < G <= (T + 63) // 64, (B, T, G)


def test_segment_plan_prefers_grids_even_over_the_cus():
    """The forward's segment count (read back from the workspace size, host
    arithmetic): for bf16 calls it picks a grid with three, else two,
    workgroups on every one of the 256 CUs when whole chunks allow it (the
    measured shapes), and bench.py's mirror of the planner agrees with the
    library on every benchmark workload."""
    import bench
    from linear_attention_rnn_amd import inputs as I

    per = 2 * (64 * 64 + 64) * 4

    def segments(B, T, H, mode, bf16):
        n = wkv6.fwd_workspace_bytes(B, T, 64 * H, H, mode, bf16)
        return n // (B * H * per) if n else 1

    assert segments(4, 4096, 16, "bidirectional", True) == 8      # 64 pairs: 512 workgroups, not 704
    assert segments(2, 4096, 16, "bidirectional", True) == 16     # 32 pairs: 512, not 704
    assert segments(2, 4096, 32, "causal", True) == 8
    assert segments(8, 4096, 16, "bidirectional", True) == 6      # 128 pairs: 768
    assert segments(8, 4096, 32, "causal", True) == 3             # 256 pairs: 768
    for w in I.WORKLOADS:
        assert segments(w.B, w.T, w.H, w.mode, w.dtype == "bf16") == bench.plan_segments(w)[0], w.name


def test_workspace_keep_bound_matches_the_header():
    import re

    with open(wkv6.HEADER) as f:
        m = re.search(r"#define WKV6_WORKSPACE_KEEP_BYTES \(\(size_t\)(\d+) << (\d+)\)", f.read())
    assert m and int(m.group(1)) << int(m.group(2)) == wkv6.WORKSPACE_KEEP_BYTES == 256 << 20
