"""C ABI checks that need no GPU: the library loads, exports every declared entry
point, and rejects invalid arguments before any HIP call."""
import ctypes
import os
import re

import pytest

import context_cross_attention_amd as cca

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    with open(os.path.join(ROOT, "include", "gdpa.h")) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gdpa_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return cca.load()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) == set(cca.EXPORTS), names
    for name in names:
        assert hasattr(lib, name), name


def P(**kw):
    base = dict(batch=2, total_tokens=10, max_seqlen=8, n_kv=4, heads=2, head_dim=64, phi=0,
                scale=0.125, dtype=1, flags=0)
    base.update(kw)
    return cca.GdpaProblem(**base)


V = ctypes.c_void_p(256)   # never dereferenced: every case fails validation first


def fwd(lib, p, ws_bytes=1 << 20, **ptrs):
    a = dict(offsets=V, q=V, k=V, v=V, residual=None, o=ctypes.c_void_p(512), lse=None, ws=V)
    a.update(ptrs)
    return lib.gdpa_fwd(ctypes.byref(p), a["offsets"], a["q"], a["k"], a["v"], a["residual"], a["o"],
                        a["lse"], a["ws"], ws_bytes, None)


def bwd(lib, p, ws_bytes=1 << 30, **ptrs):
    a = dict(offsets=V, q=V, k=V, v=V, o=V, lse=V, do=V, dq=ctypes.c_void_p(1024),
             dk=ctypes.c_void_p(2048), dv=ctypes.c_void_p(4096), ws=V)
    a.update(ptrs)
    return lib.gdpa_bwd(ctypes.byref(p), a["offsets"], a["q"], a["k"], a["v"], a["o"], a["lse"],
                        a["do"], a["dq"], a["dk"], a["dv"], a["ws"], ws_bytes, None)


INVALID, UNSUPPORTED, WS_SMALL = 1, 2, 3


@pytest.mark.parametrize("kw,status", [
    (dict(batch=0), INVALID), (dict(n_kv=0), INVALID), (dict(heads=0), INVALID),
    (dict(total_tokens=-1), INVALID), (dict(phi=7), INVALID), (dict(dtype=9), INVALID),
    (dict(scale=float("nan")), INVALID), (dict(scale=float("inf")), INVALID),
    (dict(head_dim=48), UNSUPPORTED), (dict(head_dim=256), UNSUPPORTED),
    (dict(flags=0x80), UNSUPPORTED), (dict(flags=cca.BWD_ACCUM_DQ), INVALID),
])
def test_fwd_rejects_bad_problem(lib, kw, status):
    assert fwd(lib, P(**kw)) == status


def test_fwd_rejects_bad_pointers(lib):
    assert lib.gdpa_fwd(None, V, V, V, V, None, V, None, V, 1 << 20, None) == INVALID
    assert fwd(lib, P(), offsets=None) == INVALID
    assert fwd(lib, P(), k=None) == INVALID
    assert fwd(lib, P(), o=None) == INVALID
    assert fwd(lib, P(flags=cca.FWD_RESIDUAL), residual=None) == INVALID
    assert fwd(lib, P(), o=V) == INVALID          # output aliases an input
    assert fwd(lib, P(), ws=None) == WS_SMALL
    assert fwd(lib, P(), ws_bytes=4) == WS_SMALL


def test_bwd_rejects_bad_arguments(lib):
    assert bwd(lib, P(head_dim=16)) == UNSUPPORTED
    assert bwd(lib, P(), lse=None) == INVALID      # softmax needs lse
    assert bwd(lib, P(), o=None) == INVALID
    # bf16, d = 128, n_kv <= 256: the backward sums the softmax row term itself and
    # reads no O, so o may be NULL (the call gets as far as the workspace check);
    # lse is still required.
    one_wg = dict(head_dim=128, n_kv=4)
    assert bwd(lib, P(**one_wg), o=None, ws_bytes=4) == WS_SMALL
    assert bwd(lib, P(**one_wg), o=None, lse=None) == INVALID
    assert bwd(lib, P(head_dim=128, n_kv=300), o=None) == INVALID
    assert bwd(lib, P(dtype=0, **one_wg), o=None) == INVALID   # fp32 reads O
    assert bwd(lib, P(), dk=None) == INVALID
    assert bwd(lib, P(flags=cca.FWD_RESIDUAL)) == INVALID
    assert bwd(lib, P(), dq=V, do=V) == INVALID    # in-place dQ needs the accumulate flag
    assert bwd(lib, P(), dk=ctypes.c_void_p(2048), dv=ctypes.c_void_p(2048)) == INVALID
    assert bwd(lib, P(), ws_bytes=8) == WS_SMALL


def test_weightgen_rejects_bad_arguments(lib):
    assert lib.gdpa_weightgen_fwd(0, 512, 1024, V, V, V, None) == INVALID
    assert lib.gdpa_weightgen_fwd(4, 512, 1020, V, V, V, None) == UNSUPPORTED
    assert lib.gdpa_weightgen_fwd(4, 500, 1024, V, V, V, None) == UNSUPPORTED
    assert lib.gdpa_weightgen_bwd_w(4, 512, 1024, V, None, V, None) == INVALID


def test_workspace_sizes(lib):
    assert cca.workspace_bytes(P(head_dim=48), False) == 0
    f = cca.workspace_bytes(P(batch=1000), False)
    assert f >= 4 * 1001 and f % 256 == 0
    # softmax backward keeps rowsum(dO*O) per (token, head); SiLU does not.
    soft = cca.workspace_bytes(P(total_tokens=1000, phi=0), True)
    silu = cca.workspace_bytes(P(total_tokens=1000, phi=1), True)
    assert soft - silu >= 4 * 1000 * 2
    # context rows beyond one backward work-group add the query-tile prefix sums of the
    # dQ kernel (B + 1 int32), and no fp32 dQ buffer
    big = cca.workspace_bytes(P(total_tokens=1000, phi=1, n_kv=1024, head_dim=128), True)
    assert 4 * 3 <= big - silu < 4 * 1000 * 128


def test_swa_workspace_sizes(lib):
    import ctypes
    def W(backward, **kw):
        f = dict(batch=2, total_tokens=1000, max_seqlen=1000, heads=2, head_dim=128, window=64,
                 scale=0.1, dtype=1, flags=0)
        f.update(kw)
        return int(lib.gdpa_swa_workspace_bytes(ctypes.byref(cca.SwaProblem(**f)), backward))
    assert W(0) >= 4 * 3 and W(0) % 256 == 0
    assert W(1) >= 4 * 1000 * 2       # rowsum(dO * O) per (token, head)
    assert W(1, window=0) == 0 and W(0, head_dim=48) == 0 and W(1, dtype=0) == 0


def test_pma_workspace_sizes_and_checks(lib):
    def prob(**kw):
        f = dict(batch=3, total_tokens=3000, max_seqlen=3000, heads=2, head_dim=128, seeds=32,
                 scale=0.1, dtype=1, flags=0)
        f.update(kw)
        return cca.PmaProblem(**f)

    def W(backward, **kw):
        return int(lib.gdpa_pma_workspace_bytes(ctypes.byref(prob(**kw)), backward))
    chunks = 3000 // 1024 + 3                      # upper bound on sum_b ceil(L_b / 1024)
    part = chunks * 2 * 32 * 128 * 4               # fp32 partials per (chunk, head)
    assert W(0) >= part + chunks * 2 * 32 * 2 * 4 and W(0) % 256 == 0
    assert W(1) >= part + 32 * 2 * 32 * 128 * 4     # second-level dSeeds slices
    assert W(0, seeds=0) == 0 and W(0, seeds=33) == 0 and W(0, head_dim=48) == 0
    assert W(1, dtype=0) == 0 and W(1, flags=2) == 0 and W(0, scale=float("inf")) == 0
    assert W(1, flags=cca.PMA_BWD_KV_SUM) == W(1)   # the summed backward needs nothing more
    # Invalid arguments are reported before any HIP call.
    st = lib.gdpa_pma_fwd(ctypes.byref(prob(seeds=40)), V, V, V, V, V, V, V, 1 << 30, None)
    assert st == 2
    st = lib.gdpa_pma_fwd(ctypes.byref(prob()), V, V, V, V, None, V, V, 1 << 30, None)
    assert st == 1                                  # no output
    st = lib.gdpa_pma_fwd(ctypes.byref(prob()), V, V, V, V, ctypes.c_void_p(512), V, V, 16, None)
    assert st == 3                                  # workspace too small
    st = lib.gdpa_pma_bwd(ctypes.byref(prob()), V, V, V, V, V, V, V, V, V, V, V, 1 << 30, None)
    assert st == 1                                  # outputs alias inputs
    st = lib.gdpa_pma_fwd(ctypes.byref(prob(flags=cca.PMA_BWD_KV_SUM)), V, V, V, V, ctypes.c_void_p(512), V, V,
                          1 << 30, None)
    assert st == 2                                  # the summed mode is the backward's
    ks = prob(flags=cca.PMA_BWD_KV_SUM)
    st = lib.gdpa_pma_bwd(ctypes.byref(ks), V, V, V, V, V, V, V, ctypes.c_void_p(512), ctypes.c_void_p(1024),
                          ctypes.c_void_p(2048), V, 1 << 30, None)
    assert st == 1                                  # dv must be NULL with dK + dV in dk
    st = lib.gdpa_pma_bwd(ctypes.byref(ks), V, V, ctypes.c_void_p(4096), V, V, V, V, ctypes.c_void_p(512),
                          ctypes.c_void_p(1024), None, V, 1 << 30, None)
    assert st == 1                                  # K and V must be one sequence


def test_status_strings_and_offsets_check(lib):
    assert lib.gdpa_status_str(0) == b"GDPA_OK"
    assert lib.gdpa_status_str(3) == b"GDPA_ERR_WORKSPACE_TOO_SMALL"
    assert lib.gdpa_last_hip_error() == 0
    assert cca.check_offsets([0, 3, 3, 10], 10, 7)
    assert not cca.check_offsets([0, 3, 2, 10], 10, 8)     # decreasing
    assert not cca.check_offsets([1, 3, 10], 10, 8)        # does not start at 0
    assert not cca.check_offsets([0, 3, 10], 11, 8)        # wrong total
    assert not cca.check_offsets([0, 3, 10], 10, 6)        # longer than max_seqlen
    assert cca.check_offsets([0], 0, 0)                    # empty batch
    assert not cca.check_offsets([0], 1, 0)                # empty batch with tokens


def test_group_struct_matches_header(tmp_path):
    # The ctypes mirror of gdpa_group has the C layout (size and field offsets).
    src = tmp_path / "layout.c"
    fields = [f for f, _ in cca.GdpaGroup._fields_]
    src.write_text('#include <stdio.h>\n#include <stddef.h>\n#include "gdpa.h"\nint main(void) {\n'
                   '  printf("%zu", sizeof(gdpa_group));\n'
                   + "".join(f'  printf(" %zu", offsetof(gdpa_group, {f}));\n' for f in fields) + "  return 0;\n}\n")
    exe = tmp_path / "layout"
    import subprocess
    subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    got = [int(x) for x in subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split()]
    want = [ctypes.sizeof(cca.GdpaGroup)] + [getattr(cca.GdpaGroup, f).offset for f in fields]
    assert got == want


def test_grouped_checks_every_group_first(lib):
    arr = (cca.GdpaGroup * 3)()
    for i, d in enumerate((32, 64, 128)):
        arr[i].problem = P(head_dim=d)
        arr[i].offsets, arr[i].q, arr[i].k, arr[i].v, arr[i].o = 256, 256, 256, 256, 512 + i * 64
    one = int(lib.gdpa_workspace_bytes(ctypes.byref(P()), 0))
    total = int(lib.gdpa_grouped_workspace_bytes(3, arr, 0))
    assert total >= 3 * one and total % 256 == 0
    assert int(lib.gdpa_grouped_workspace_bytes(3, arr, 1)) > 0
    assert lib.gdpa_fwd_grouped(3, arr, V, total - 1, None) == WS_SMALL
    assert lib.gdpa_fwd_grouped(0, arr, V, total, None) == INVALID
    arr[2].problem = P(head_dim=48)                 # the last group is unsupported:
    assert lib.gdpa_fwd_grouped(3, arr, V, 1 << 30, None) == UNSUPPORTED   # nothing launched
    assert int(lib.gdpa_grouped_workspace_bytes(3, arr, 0)) == 0
    arr[2].problem = P(head_dim=128)
    arr[1].o = None                                 # a group without its output
    assert lib.gdpa_fwd_grouped(3, arr, V, 1 << 30, None) == INVALID
    arr[1].o = 2048
    arr[2].o = 2048                                 # two groups writing one buffer
    assert lib.gdpa_fwd_grouped(3, arr, V, 1 << 30, None) == INVALID
    arr[2].o = arr[0].q                             # a group writing another's input
    assert lib.gdpa_fwd_grouped(3, arr, V, 1 << 30, None) == INVALID
    arr[2].o = 4096
    arr[0].dq = None                                # backward needs dq
    assert lib.gdpa_bwd_grouped(3, arr, V, 1 << 30, None) == INVALID


def noalloc(lib, p, **ptrs):
    a = dict(offsets=V, q=V, k=V, v=V, o=V, lse=V, do=V, dq=ctypes.c_void_p(1024),
             dk=ctypes.c_void_p(2048), dv=ctypes.c_void_p(4096))
    a.update(ptrs)
    return lib.gdpa_bwd_noalloc(ctypes.byref(p), a["offsets"], a["q"], a["k"], a["v"], a["o"], a["lse"],
                                a["do"], a["dq"], a["dk"], a["dv"], None)


def test_bwd_noalloc_checks_before_any_device_call(lib):
    # The allocation-free backward validates like gdpa_bwd, and rejects a problem whose
    # workspace exceeds the per-GPU scratch, all before touching the device.
    assert cca.NOALLOC_SCRATCH_BYTES == 64 << 20
    assert noalloc(lib, P(head_dim=48)) == UNSUPPORTED
    assert noalloc(lib, P(), lse=None) == INVALID
    assert noalloc(lib, P(), dk=None) == INVALID
    assert noalloc(lib, P(), dq=V, do=V) == INVALID
    assert lib.gdpa_bwd_noalloc(None, V, V, V, V, V, V, V, V, V, V, None) == INVALID
    # softmax keeps 4 bytes of row dots per (token, head): 2^24 rows no longer fit with the
    # sample order next to them; the elementwise maps need only the order.
    big = P(batch=4, total_tokens=1 << 22, max_seqlen=1 << 22, heads=4, head_dim=32, phi=0)
    assert cca.workspace_bytes(big, True) > cca.NOALLOC_SCRATCH_BYTES
    assert noalloc(lib, big) == WS_SMALL
    fits = P(batch=4, total_tokens=(1 << 22) - 4096, max_seqlen=1 << 22, heads=4, head_dim=32, phi=0)
    assert cca.workspace_bytes(fits, True) <= cca.NOALLOC_SCRATCH_BYTES


def test_fwd_block_checks(lib):
    def blk(p, o=ctypes.c_void_p(512), y=ctypes.c_void_p(768), x=V):
        return lib.gdpa_fwd_block(ctypes.byref(p), V, x, V, V, o, y, None, V, 1 << 20, None)
    assert blk(P(flags=cca.FWD_RESIDUAL)) == UNSUPPORTED   # the block is already residual
    assert blk(P(), y=None) == INVALID
    assert blk(P(), y=V) == INVALID                        # y aliases x (and k, v)
    assert blk(P(), y=ctypes.c_void_p(512)) == INVALID     # y aliases o
    assert blk(P(), o=V) == INVALID                        # o aliases an input
    assert blk(P(head_dim=48)) == UNSUPPORTED
