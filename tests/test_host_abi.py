"""Host-side checks of the C ABI (no GPU needed).

The library must load, export every function include/moba.h declares, and
reject bad arguments on the host before any launch.  Only host-only entry
points and validation paths are called here.
"""
import ctypes
import os
import re

import pytest

import block_sparse_long_key_amd as moba
import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moba.h")

OK, INVALID, UNSUPPORTED, WS_SMALL = 0, 1, 2, 3


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(moba.library_path()):
        import __graft_entry__
        __graft_entry__.build()
    return moba._load()


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moba_[a-z_0-9]+)\s*\(", src)))


def test_exports_every_declared_function(lib):
    names = _declared()
    assert "moba_attn_fwd" in names and "moba_route_topk" in names
    for n in names:
        assert hasattr(lib, n), f"{n} not exported"
    assert lib.moba_abi_version() == 3
    assert lib.moba_status_string(0) == b"ok"
    assert lib.moba_status_string(WS_SMALL) == b"workspace too small"


def test_debug_build_exports_and_release_has_no_checks(lib):
    """The bounds-checking build exports every declared function under the
    same ABI; the release build answers moba_debug_violations with
    MOBA_ERR_UNSUPPORTED and leaves the flags alone (no device access)."""
    from block_sparse_long_key_amd import build as mbuild
    if not os.path.exists(mbuild.DEBUG_LIB):
        pytest.skip("the debug library is not built")
    dbg = ctypes.CDLL(mbuild.DEBUG_LIB)
    for n in _declared():
        assert hasattr(dbg, n), f"{n} not exported by the debug build"
    assert dbg.moba_abi_version() == lib.moba_abi_version()
    lib.moba_debug_violations.argtypes = [ctypes.c_void_p]
    lib.moba_debug_violations.restype = ctypes.c_int32
    f = ctypes.c_uint32(7)
    assert lib.moba_debug_violations(ctypes.byref(f)) == UNSUPPORTED
    assert f.value == 7


def _shape(batch=1, seq=1024, heads=2, d=64, B=64, K=4, dtype=1, cu=None):
    if cu is not None:
        arr = (ctypes.c_int32 * len(cu))(*cu)
        sh = moba._Shape(1, cu[-1], heads, d, ctypes.cast(arr, ctypes.POINTER(ctypes.c_int32)),
                         len(cu) - 1, B, K, dtype)
        sh._keep = arr
        return sh
    return moba._Shape(batch, seq, heads, d, None, 0, B, K, dtype)


def test_total_blocks_and_workspace(lib):
    assert lib.moba_total_blocks(ctypes.byref(_shape(batch=2, seq=1000, B=64))) == 2 * 16
    sh = _shape(cu=[0, 100, 100, 300], B=64)
    assert lib.moba_total_blocks(ctypes.byref(sh)) == 2 + 0 + 4
    assert lib.moba_attn_fwd_workspace_bytes(ctypes.byref(_shape(K=1))) == 0
    ws = lib.moba_attn_fwd_workspace_bytes(ctypes.byref(_shape()))
    # at least the partial outputs: tokens * heads * k * (d * 2 + 4)
    assert ws >= 1024 * 2 * 4 * (64 * 2 + 4)
    s = workloads.spec("H")
    big = lib.moba_attn_fwd_workspace_bytes(ctypes.byref(_shape(2, 65536, 16, 64, 128, 8)))
    assert big >= s.batch * s.seq * s.heads * s.top_k * (s.head_dim * 2 + 4)


def test_large_blocks_attend_as_128_key_blocks(lib):
    # MoBA-256 / MoBA-512 shapes are accepted; their attention workspace is
    # that of 128-key blocks with top_k * B / 128 slots plus the expanded
    # selection, so even top_k = 1 (own block only) has routed lists
    for B, K in ((256, 4), (512, 2), (256, 1)):
        sh = _shape(batch=2, seq=4096, B=B, K=K)
        assert lib.moba_total_blocks(ctypes.byref(sh)) == 2 * 4096 // B
        ws = lib.moba_attn_fwd_workspace_bytes(ctypes.byref(sh))
        ref = lib.moba_attn_fwd_workspace_bytes(ctypes.byref(_shape(batch=2, seq=4096, B=128,
                                                                   K=K * B // 128)))
        assert ws >= ref + 2 * 4096 * sh.heads * (K * B // 128) * 4
        assert lib.moba_attn_bwd_workspace_bytes(ctypes.byref(sh)) > 0


@pytest.mark.parametrize("kw,code", [
    (dict(d=96), UNSUPPORTED), (dict(B=32), UNSUPPORTED), (dict(B=1024), UNSUPPORTED),
    (dict(B=256, K=9), UNSUPPORTED), (dict(dtype=0, B=512), UNSUPPORTED),
    (dict(K=0), INVALID), (dict(K=33), UNSUPPORTED), (dict(dtype=7), INVALID),
    (dict(heads=0), INVALID),
    (dict(dtype=0, d=128, B=128, K=17), UNSUPPORTED),   # 17 x 2 sub-blocks > 32 slots
    (dict(cu=[0, 10, 5]), INVALID), (dict(cu=[1, 10]), INVALID),
    (dict(cu=list(range(0, 2000, 10)) + [1990 + 16385 * 64], B=64), UNSUPPORTED),  # 16385 blocks in the last group
    (dict(cu=list(range(0, 2000, 10)) + [1995, 1990]), INVALID),  # decreasing past group 0
    (dict(seq=1 << 26, heads=2), UNSUPPORTED),              # tokens x heads = 2^27
    (dict(seq=16384 * 64 + 1, B=64), UNSUPPORTED),          # 16385 blocks in a sequence
])
def test_bad_shapes_rejected_on_host(lib, kw, code):
    sh = _shape(**kw)
    p = ctypes.c_void_p(16 * 1024)          # never dereferenced: validation fails first
    rc = lib.moba_route_topk(ctypes.byref(sh), p, p, p, p, 1 << 30, None)
    assert rc == code
    assert lib.moba_total_blocks(ctypes.byref(sh)) == -1
    assert lib.moba_attn_fwd_workspace_bytes(ctypes.byref(sh)) == 0


def test_fp32_d128_attends_64_key_sub_blocks(lib):
    """fp32 at d = 128 attends 64-key blocks: B = 128 / 256 selections are
    expanded to 2 / 4 sub-blocks, so the workspace is that of B = 64 with
    top_k * B / 64 slots plus the expanded selection."""
    for B, K in ((128, 16), (128, 1), (256, 8)):
        sh = _shape(batch=2, seq=4096, d=128, B=B, K=K, dtype=0)
        assert lib.moba_total_blocks(ctypes.byref(sh)) == 2 * 4096 // B
        ws = lib.moba_attn_fwd_workspace_bytes(ctypes.byref(sh))
        ref = lib.moba_attn_fwd_workspace_bytes(ctypes.byref(_shape(batch=2, seq=4096, d=128, B=64,
                                                                   K=K * B // 64, dtype=0)))
        assert ws >= ref + 2 * 4096 * sh.heads * (K * B // 64) * 4
        assert lib.moba_attn_bwd_workspace_bytes(ctypes.byref(sh)) > 0
    p = ctypes.c_void_p(16 * 1024)
    sh = _shape(batch=2, seq=4096, d=128, B=128, K=8, dtype=0)
    # BLASST takes whole blocks only
    assert lib.moba_attn_fwd_blasst(ctypes.byref(sh), p, p, p, p, ctypes.c_float(0.0),
                                    ctypes.c_float(0.5), p, None, None, p, 1 << 40, None) == UNSUPPORTED
    # and so does its backward
    assert lib.moba_attn_bwd_blasst(ctypes.byref(sh), p, p, p, p, ctypes.c_float(0.0), p, p, p,
                                    ctypes.c_void_p(1 << 20), ctypes.c_void_p(1 << 21),
                                    ctypes.c_void_p(1 << 22), p, 1 << 40, None) == UNSUPPORTED


def test_blasst_kept_idx_checked_on_the_host(lib):
    """kept_idx must be 16-byte aligned and must not be idx; refused
    before any launch (no device memory is touched)."""
    p = ctypes.c_void_p(16 * 1024)
    sh = _shape(batch=1, seq=1024, B=64, K=4)
    for bad in (ctypes.c_void_p(16 * 1024 + 4), p):
        assert lib.moba_attn_fwd_blasst(ctypes.byref(sh), p, p, p, p, ctypes.c_float(0.0),
                                        ctypes.c_float(0.5), p, None, bad, p, 1 << 40,
                                        None) == INVALID


def test_largest_accepted_shapes(lib):
    # 16384 blocks in one sequence and 63 * 2^21 < 2^27 token-heads are
    # accepted on the host
    sh = _shape(seq=16384 * 128, heads=63, B=128, K=8)
    assert lib.moba_total_blocks(ctypes.byref(sh)) == 16384
    assert lib.moba_attn_fwd_workspace_bytes(ctypes.byref(sh)) > 0


def _one_group_sums(lib, lens, B=64, K=4, heads=2, d=64):
    """Workspace of a many-sequence call vs the calls of its groups of 64."""
    cu = [0]
    for L in lens:
        cu.append(cu[-1] + L)
    sh = _shape(cu=cu, B=B, K=K, heads=heads, d=d)
    parts = []
    for g in range(0, len(lens), 64):
        sub = lens[g:g + 64]
        c = [0]
        for L in sub:
            c.append(c[-1] + L)
        parts.append(_shape(cu=c, B=B, K=K, heads=heads, d=d))
    return sh, parts


@pytest.mark.parametrize("nseq", [64, 65, 200])
def test_many_sequences_run_in_groups_of_64(lib, nseq):
    """More varlen sequences than one launch table holds (MOBA_MAX_SEQS) are
    accepted: the call runs them as groups of 64, so block counts add up, the
    attention workspaces hold one region per group and the routing
    workspace is the largest group's."""
    lens = [(37 * i) % 300 for i in range(nseq)]
    sh, parts = _one_group_sums(lib, lens)
    nb = sum((L + 63) // 64 for L in lens)
    assert lib.moba_total_blocks(ctypes.byref(sh)) == nb
    for f in (lib.moba_attn_fwd_workspace_bytes, lib.moba_attn_bwd_workspace_bytes):
        assert f(ctypes.byref(sh)) == sum(f(ctypes.byref(p)) for p in parts)
    r = lib.moba_route_topk_workspace_bytes
    assert r(ctypes.byref(sh)) == max(r(ctypes.byref(p)) for p in parts)
    assert lib.moba_key_conv_bwd_workspace_bytes(ctypes.byref(sh), 3) >= nb * 2 * 64 * 3 * 4
    # a uniform batch of more than 64 rows too
    assert lib.moba_total_blocks(ctypes.byref(_shape(batch=130, seq=100, B=64))) == 260


def test_many_sequence_attention_workspace_is_checked_whole(lib):
    lens = [100] * 130
    sh, parts = _one_group_sums(lib, lens)
    need = lib.moba_attn_fwd_workspace_bytes(ctypes.byref(sh))
    p = ctypes.c_void_p(1 << 20)
    assert lib.moba_attn_index(ctypes.byref(sh), p, p, need - 256, None) == WS_SMALL
    assert lib.moba_attn_bwd(ctypes.byref(sh), p, p, p, p, ctypes.c_float(0.0), p, p, p,
                             ctypes.c_void_p(2 << 20), ctypes.c_void_p(3 << 20),
                             ctypes.c_void_p(4 << 20), p,
                             lib.moba_attn_bwd_workspace_bytes(ctypes.byref(sh)) - 256,
                             None) == WS_SMALL


def test_route_workspace(lib):
    """The router's workspace holds the split centroids: bf16 high and low
    parts [block][head][d] and fp32 squared norms [block][head]."""
    def a256(x):
        return (x + 255) // 256 * 256
    for d in (64, 128):
        sh = _shape(batch=2, seq=1000, heads=3, d=d, B=64)
        rows = 2 * 16 * 3
        assert lib.moba_route_topk_workspace_bytes(ctypes.byref(sh)) == \
            2 * a256(rows * d * 2) + a256(rows * 4)
    assert lib.moba_route_topk_workspace_bytes(ctypes.byref(_shape(heads=0))) == 0
    sh = _shape()
    good = ctypes.c_void_p(1 << 20)
    odd = ctypes.c_void_p((1 << 20) + 64)
    need = lib.moba_route_topk_workspace_bytes(ctypes.byref(sh))
    assert lib.moba_route_topk(ctypes.byref(sh), good, good, good, None, need, None) == INVALID
    assert lib.moba_route_topk(ctypes.byref(sh), good, good, good, odd, need, None) == INVALID
    assert lib.moba_route_topk(ctypes.byref(sh), good, good, good, good, need - 1, None) == WS_SMALL


def test_null_misaligned_and_small_workspace_rejected(lib):
    sh = _shape()
    good = ctypes.c_void_p(1 << 20)
    odd = ctypes.c_void_p((1 << 20) + 4)
    assert lib.moba_centroids(ctypes.byref(sh), None, good, None) == INVALID
    assert lib.moba_centroids(ctypes.byref(sh), odd, good, None) == INVALID
    assert lib.moba_route_topk(None, good, good, good, good, 1 << 30, None) == INVALID
    need = lib.moba_attn_fwd_workspace_bytes(ctypes.byref(sh))
    rc = lib.moba_attn_fwd(ctypes.byref(sh), good, good, good, good, 0.0, good, None, good,
                           need - 1, None)
    assert rc == WS_SMALL
    rc = lib.moba_attn_fwd(ctypes.byref(sh), good, good, good, good, 0.0, good, None,
                           ctypes.c_void_p((1 << 20) + 16), need, None)
    assert rc == INVALID                    # workspace must be 256-byte aligned
    # conv: width and mode checks, aliasing
    assert lib.moba_key_conv(ctypes.byref(sh), good, good, 9, 0, ctypes.c_void_p(2 << 20),
                             None, None) == UNSUPPORTED
    assert lib.moba_key_conv(ctypes.byref(sh), good, good, 3, 5, ctypes.c_void_p(2 << 20),
                             None, None) == INVALID
    assert lib.moba_key_conv(ctypes.byref(sh), good, good, 3, 0, good, None, None) == INVALID


def test_python_binding_refuses_cpu_tensors():
    import torch
    q = torch.zeros(1, 64, 1, 64, dtype=torch.bfloat16)
    with pytest.raises(moba.MobaError):
        moba.moba_centroids(q, 64)


C_CALLER = r"""
#include "moba.h"
#include <stdio.h>
int main(void) {
    int32_t cu[3] = {0, 1000, 1300};
    moba_shape sh = {0};
    sh.batch = 1; sh.seq = 1300; sh.heads = 2; sh.head_dim = 64;
    sh.cu_seqlens = cu; sh.num_seqs = 2; sh.block_size = 128; sh.top_k = 4;
    sh.dtype = MOBA_BF16;
    /* a null q is refused on the host, before any device work */
    moba_status st = moba_centroids(&sh, NULL, (float *)256, NULL);
    printf("%d %lld %d %s\n", moba_abi_version(), (long long)moba_total_blocks(&sh),
           moba_attn_fwd_workspace_bytes(&sh) > 0, moba_status_string(st));
    return 0;
}
"""


def test_header_compiles_as_c_and_links(lib, tmp_path):
    """A plain C99 program includes moba.h, links the library and calls the
    host-only entry points (no torch, no GPU)."""
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None or not os.path.isdir("/opt/rocm/include"):
        pytest.skip("gcc or the ROCm headers are not available")
    src = tmp_path / "caller.c"
    src.write_text(C_CALLER)
    exe = tmp_path / "caller"
    libdir = os.path.dirname(moba.library_path())
    libname = os.path.basename(moba.library_path())[3:-3]
    subprocess.run([gcc, "-std=c99", "-Wall", "-Werror=implicit-function-declaration",
                    "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
                    "-I", "/opt/rocm/include", str(src), "-L", libdir, f"-l{libname}",
                    f"-Wl,-rpath,{libdir}", "-o", str(exe)], check=True, capture_output=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split(None, 3)
    assert int(out[0]) == lib.moba_abi_version()
    assert int(out[1]) == 11                  # ceil(1000/128) + ceil(300/128)
    assert out[2] == "1"
    assert out[3].strip() == lib.moba_status_string(INVALID).decode()


def test_route_noalloc_refuses_shapes_beyond_its_scratch(lib):
    """The no-allocation routing call checks its fixed scratch size on the
    host, before any launch (bf16: 4 d + 4 bytes per (block, head) row)."""
    fake = ctypes.c_void_p(1 << 20)            # never dereferenced: refused first
    # 2 x 262144 tokens, 64 heads, B = 64: 8192 blocks x 64 heads = 524288 rows
    big = _shape(batch=2, seq=262144, heads=64, d=64, B=64, K=8)
    need = lib.moba_route_topk_workspace_bytes(ctypes.byref(big))
    assert need > 32 << 20
    assert lib.moba_route_topk_noalloc(ctypes.byref(big), fake, fake, fake, None) == WS_SMALL
    # more sequences than one launch group: the second group alone (one
    # 262144-token sequence of 64 heads) is too big, and the call is refused
    # before the first group is launched (no HIP call is made at all here)
    cu = [128 * n for n in range(65)] + [128 * 64 + 262144]
    multi = _shape(cu=cu, heads=64, d=64, B=64, K=8)
    assert lib.moba_route_topk_noalloc(ctypes.byref(multi), fake, fake, fake, None) == WS_SMALL
    # the same for moba_route_topk with a caller's workspace that holds the
    # first group's routing data but not the second's
    small = lib.moba_route_topk_workspace_bytes(ctypes.byref(_shape(cu=cu[:65], heads=64, d=64, B=64, K=8)))
    assert 0 < small < lib.moba_route_topk_workspace_bytes(ctypes.byref(multi))
    wsp = ctypes.c_void_p(1 << 24)             # 256-byte aligned, never dereferenced
    assert lib.moba_route_topk(ctypes.byref(multi), fake, fake, fake, wsp, small, None) == WS_SMALL
    # and a multi-group attention call without a workspace
    assert lib.moba_attn_fwd(ctypes.byref(multi), fake, fake, fake, fake, ctypes.c_float(0.0), fake,
                             None, None, 0, None) == INVALID
    # invalid arguments are still refused as such
    assert lib.moba_route_topk_noalloc(ctypes.byref(_shape()), None, fake, fake, None) == INVALID
    assert lib.moba_route_topk_noalloc(ctypes.byref(_shape(d=96)), fake, fake, fake, None) == UNSUPPORTED
