"""Host-side checks of the C-ABI library: it loads, exports every entry point
that include/arl2.h declares, and rejects bad arguments before launching
anything. None of these calls reaches the GPU (validation fails first), so
they run without one. Also covers the pass sequencer's host logic."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "arl2.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(arl2_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def arl2():
    from hybrid_linear_memory_amd import arl2 as mod
    return mod


def test_every_declared_symbol_is_exported(arl2):
    names = _declared()
    assert len(names) >= 12
    lib = ctypes.CDLL(arl2._LIB_PATH)
    for n in names:
        assert hasattr(lib, n), f"{n} declared in arl2.h but not exported"
    assert set(names) == set(arl2.SIGNATURES), "binding signatures out of sync with arl2.h"


def test_version_and_status_strings(arl2):
    assert arl2.abi_version() == arl2.ABI_VERSION == 2
    hdr = open(os.path.join(os.path.dirname(arl2._LIB_PATH), "..", "include", "arl2.h")).read()
    assert re.search(r"#define ARL2_ABI_VERSION (\d+)", hdr).group(1) == str(arl2.ABI_VERSION)
    for code, name in arl2.STATUS_NAMES.items():
        assert arl2.status_string(code) == name
    assert arl2.status_string(99) == "ARL2_E_UNKNOWN"


def test_workspace_sizes(arl2):
    s = arl2.Shape(1, 12, 1560, 128, arl2.BF16)
    act = 1 * 12 * 1560 * 128 * 2
    assert arl2.workspace_bytes(s, arl2.OP_READ) >= 12 * 128 * 128 * 2
    # the bf16 commit and the one-launch clean pass: per (video, head, 32 state
    # columns) one fp32 sum of 128 x 32 per token part and one 8-byte counter.
    # The clean pass takes two parts; the commit alone at most as many as fill
    # 256 compute units (at least 2, at most 8, and at least eight 32-token
    # slices per part where the frame has them), then the fewest that keep
    # each wave's slice count (here 49 slices: 5 parts of <= 10 slices and 4
    # of <= 13 both give two per wave, so 4); the commit from given K', V' sums
    # fp32 partials of its token chunks
    def parts_ws(cblocks, parts):
        return cblocks * parts * 4096 * 4 + (cblocks * 8 + 255) // 256 * 256
    cblocks = 1 * 12 * 4
    assert arl2.workspace_bytes(s, arl2.OP_COMMIT) == parts_ws(cblocks, 4)
    assert arl2.workspace_bytes(s, arl2.OP_CLEAN_PASS_PREPARED) == parts_ws(cblocks, 2)
    eight = arl2.Shape(8, 12, 1560, 128, arl2.BF16)
    assert arl2.workspace_bytes(eight, arl2.OP_COMMIT) == parts_ws(8 * 12 * 4, 2)
    short = arl2.Shape(1, 2, 100, 128, arl2.BF16)         # 4 slices: two parts
    assert arl2.workspace_bytes(short, arl2.OP_COMMIT) == parts_ws(2 * 4, 2)
    three = arl2.Shape(1, 1, 768, 128, arl2.BF16)         # 24 slices: 3 parts of 8
    assert arl2.workspace_bytes(three, arl2.OP_COMMIT) == parts_ws(4, 3)
    most = arl2.Shape(1, 1, 4000, 128, arl2.BF16)         # 125 slices: 8 parts of <= 16
    assert arl2.workspace_bytes(most, arl2.OP_COMMIT) == parts_ws(4, 8)
    assert arl2.workspace_bytes(s, arl2.OP_STATE_COMMIT) > 0
    assert arl2.workspace_bytes(s, arl2.OP_CLEAN_PASS) == max(
        arl2.workspace_bytes(s, arl2.OP_READ), arl2.workspace_bytes(s, arl2.OP_COMMIT))
    # the plain grid at 12 heads x 1560 tokens: no workspace
    assert arl2.workspace_bytes(s, arl2.OP_READ_PREPARED) == 0
    assert arl2.workspace_bytes(s, arl2.OP_READ) == 12 * 128 * 128 * 2
    # split-key read (4 heads x 4096 tokens: 128 query blocks of 64 key tiles):
    # one 8-byte counter per query block, then two slots per workgroup (256)
    # of 8 x 2048 output floats and 512 (maximum, sum) pairs; the one-call
    # read puts M^T first
    s4 = arl2.Shape(1, 4, 4096, 128, arl2.BF16)
    split = (128 * 8 + 255) // 256 * 256 + 2 * 256 * (8 * 2048 + 1024) * 4
    assert arl2.workspace_bytes(s4, arl2.OP_READ_PREPARED) == split
    assert arl2.workspace_bytes(s4, arl2.OP_READ) == 4 * 128 * 128 * 2 + split
    # no split where the plain grid fills the chip, or at most 10% would be won
    for B, H, T in ((8, 12, 1560), (1, 3, 300), (1, 6, 4096), (1, 8, 3000)):
        assert arl2.workspace_bytes(arl2.Shape(B, H, T, 128, arl2.BF16),
                                    arl2.OP_READ_PREPARED) == 0, (B, H, T)
    for B, H, T in ((2, 2, 4096), (1, 5, 4000), (1, 3, 8192), (1, 1, 16384), (1, 40, 1560),
                    (1, 12, 3600)):
        assert arl2.workspace_bytes(arl2.Shape(B, H, T, 128, arl2.BF16),
                                    arl2.OP_READ_PREPARED) > 0, (B, H, T)
    assert arl2.workspace_bytes(s, 17) == 0
    assert arl2.workspace_bytes(arl2.Shape(0, 1, 1, 128), arl2.OP_READ) == 0
    f = arl2.Shape(1, 1, 64, 16, arl2.F32)
    assert arl2.workspace_bytes(f, arl2.OP_STATE_COMMIT) == 64 * 16 * 4
    # token-level access: Q', K', V', o_intra, then (bf16) per 64-token chunk of
    # each head W [64, D] bf16, U [64, D] fp32 and Pq [64, 64] bf16
    chunks = 12 * ((1560 + 63) // 64)
    assert arl2.workspace_bytes(s, arl2.OP_TOKEN_LEVEL) == 4 * act + chunks * 64 * (
        128 * 2 + 128 * 4 + 64 * 2)
    assert arl2.workspace_bytes(f, arl2.OP_TOKEN_LEVEL) == 4 * 64 * 16 * 4


A = 1 << 20     # fake, 16-byte aligned "device" addresses: validation fails before any use
B = 2 << 20


def _st(arl2, name, *args):
    return arl2.raw_call(name, *args)


def test_null_shape_dtype_layout_errors(arl2):
    good = arl2.Shape(1, 2, 64, 128, arl2.BF16)
    cs = arl2.c_shape
    assert _st(arl2, "arl2_intra_attn", None, A, A, A, B, None) == 1
    assert _st(arl2, "arl2_intra_attn", cs(good), None, A, A, B, None) == 1
    assert "'q'" in arl2.last_error()
    # bf16 runs at D in {16, 32, 64, 128}: an unsupported D is a shape error, a
    # supported one reaches the alias check (o over q) before any launch
    assert _st(arl2, "arl2_intra_attn", cs(arl2.Shape(1, 2, 64, 48, arl2.BF16)), A, A, A, B,
               None) == 2
    for D in (16, 32, 64):
        assert _st(arl2, "arl2_intra_attn", cs(arl2.Shape(1, 2, 64, D, arl2.BF16)), A, B, B, A,
                   None) == 5
    assert _st(arl2, "arl2_intra_attn", cs(arl2.Shape(1, 2, 0, 128, arl2.BF16)), A, A, A, B,
               None) == 2
    assert _st(arl2, "arl2_intra_attn", cs(arl2.Shape(1, 2, 64, 48, arl2.F32)), A, A, A, B,
               None) == 2
    assert _st(arl2, "arl2_intra_attn", cs(arl2.Shape(1, 2, 64, 128, 7)), A, A, A, B, None) == 3
    assert _st(arl2, "arl2_intra_attn", cs(arl2.Shape(1, 2, 64, 128, arl2.BF16, -1.0)), A, A, A,
               B, None) == 2
    assert _st(arl2, "arl2_intra_attn", cs(good), A + 2, A, A, B, None) == 4
    assert _st(arl2, "arl2_intra_attn", cs(good), A, A, A, A + 64, None) == 5
    assert _st(arl2, "arl2_intra_attn", cs(arl2.Shape(4096, 64, 4096, 128)), A, A, A, B,
               None) == 2


def test_alias_and_workspace_errors(arl2):
    # float32: the commit maps K and V into its workspace, so every commit call
    # below fails validation before anything could be launched
    s = arl2.Shape(1, 2, 1560, 128, arl2.BF16)
    f = arl2.Shape(1, 2, 1560, 64, arl2.F32)
    cs = arl2.c_shape
    assert arl2.workspace_bytes(f, arl2.OP_COMMIT) > 0
    S1, S2, WS = 8 << 20, 16 << 20, 32 << 20
    need = arl2.workspace_bytes(f, arl2.OP_COMMIT)
    # S_prev == S_next
    assert _st(arl2, "arl2_commit", cs(f), A, A, A, A, A, A, S1, S1, WS, need, None) == 5
    # overlapping by one element
    assert _st(arl2, "arl2_commit", cs(f), A, A, A, A, A, A, S1, S1 + 16, WS, need, None) == 5
    # workspace missing / too small
    assert _st(arl2, "arl2_commit", cs(f), A, A, A, A, A, A, S1, S2, None, 0, None) == 6
    assert _st(arl2, "arl2_commit", cs(f), A, A, A, A, A, A, S1, S2, WS, need - 1, None) == 6
    assert "needed" in arl2.last_error()
    # read outputs overlapping inputs
    rneed = arl2.workspace_bytes(s, arl2.OP_READ)
    assert _st(arl2, "arl2_read", cs(s), A, B, B, B, S1, A, None, None, WS, rneed, None) == 5
    # one-launch clean pass: S_next aliasing S_prev; float32 (read and commit
    # one after the other in the workspace): missing workspace
    cneed = arl2.workspace_bytes(s, arl2.OP_CLEAN_PASS_PREPARED)
    assert _st(arl2, "arl2_clean_pass_prepared", cs(s), A, A, A, A, None, A, A, A, A, S1, S1,
               None, B, None, None, WS, cneed, None) == 5
    assert arl2.workspace_bytes(f, arl2.OP_CLEAN_PASS_PREPARED) > 0
    assert _st(arl2, "arl2_clean_pass_prepared", cs(f), A, A, A, A, None, A, A, A, A, S1, S2,
               None, B, None, None, None, 0, None) == 6
    # the next map wanted without phi_q
    assert _st(arl2, "arl2_clean_pass_prepared", cs(s), A, A, A, A, None, A, A, A, A, S1, S2,
               B + 4096, B, None, None, WS, cneed, None) == 1
    # token-level access: S_next aliasing S_prev, missing alpha, workspace short,
    # an output over an input
    tneed = arl2.workspace_bytes(s, arl2.OP_TOKEN_LEVEL)
    assert _st(arl2, "arl2_token_clean_pass", cs(s), A, A, A, A, A, A, A, A, S1, S1, B, None,
               None, WS, tneed, None) == 5
    assert _st(arl2, "arl2_token_clean_pass", cs(s), A, A, A, A, A, A, A, None, S1, S2, B, None,
               None, WS, tneed, None) == 1
    assert _st(arl2, "arl2_token_read", cs(s), A, A, A, A, A, A, A, S1, B, None, None, WS,
               tneed - 1, None) == 6
    assert _st(arl2, "arl2_token_read", cs(s), A, A, A, A, A, A, A, S1, A, None, None, WS, tneed,
               None) == 5
    # training side: workspace short, dS_prev over dS_next, outputs overlapping
    cb = arl2.workspace_bytes(s, arl2.OP_COMMIT_BACKWARD)
    assert _st(arl2, "arl2_commit_backward", cs(s), A, A, A, A, A, A, S1, S2, B, B + (2 << 20),
               B + (4 << 20), B + (5 << 20), B + (6 << 20), B + (7 << 20), S2, 0, WS, cb - 1,
               None) == 6
    assert _st(arl2, "arl2_commit_backward", cs(s), A, A, A, A, A, A, S1, S2, B, B + (2 << 20),
               B + (4 << 20), B + (5 << 20), B + (6 << 20), B + (7 << 20), S2, 0, WS, cb,
               None) == 5
    rb = arl2.workspace_bytes(s, arl2.OP_READ_BACKWARD)
    assert _st(arl2, "arl2_read_backward", cs(s), A, A, A, A, S1, A, None, A, B, B, B + (4 << 20),
               B + (6 << 20), S2, 0, WS, rb, None) == 5
    # the rows' log-sum-exp (optional input) must not overlap an output
    ab = arl2.workspace_bytes(s, arl2.OP_INTRA_ATTN_BACKWARD)
    assert _st(arl2, "arl2_intra_attn_backward", cs(s), A, A, A, A, B, A, B, B + (4 << 20),
               B + (6 << 20), 0, WS, ab, None) == 5
    assert _st(arl2, "arl2_intra_attn_lse", cs(s), A, A, A, B, B, None) == 5
    assert _st(arl2, "arl2_state_scan", cs(f), 0, A, A, A, A, A, A, S1, S2, WS, need, None) == 2
    # S_next over an input or the workspace (state commit, commit, clean pass)
    sneed = arl2.workspace_bytes(s, arl2.OP_STATE_COMMIT)
    assert sneed > 0
    assert _st(arl2, "arl2_state_commit", cs(s), A, A, A, A, S1, WS, WS, sneed, None) == 5
    assert _st(arl2, "arl2_state_commit", cs(s), B, A, A, A, S1, B + 4096, WS, sneed,
               None) == 5
    assert _st(arl2, "arl2_commit", cs(f), A, A, A, A, A, A, S1, A + 4096, WS, need, None) == 5
    assert _st(arl2, "arl2_commit", cs(f), A, A, A, A, A, B, S1, B, WS, need, None) == 5
    clneed = arl2.workspace_bytes(s, arl2.OP_CLEAN_PASS)
    for phi_k, alpha in ((S2, A), (A, S2)):
        assert _st(arl2, "arl2_clean_pass", cs(s), A, A, A, A, phi_k, A, A, alpha, S1, S2, B,
                   None, None, WS, clneed, None) == 5
    # token-level and training calls keep bf16 at D = 128
    s64 = arl2.Shape(1, 2, 300, 64, arl2.BF16)
    assert _st(arl2, "arl2_token_read", cs(s64), A, A, A, A, A, A, A, S1, B, None, None, WS,
               1 << 20, None) == 2
    assert "D = 128" in arl2.last_error()
    assert _st(arl2, "arl2_intra_attn_lse", cs(s64), A, A, A, B, S1, None) == 2
    assert _st(arl2, "arl2_intra_attn_backward", cs(s64), A, A, A, A, None, A, B, B + (4 << 20),
               B + (6 << 20), 0, WS, 1 << 20, None) == 2
    # fullkv: n_kv beyond capacity
    assert _st(arl2, "arl2_fullkv_attn", cs(s), A, B, S1, 200, 100, WS, None) == 2


def test_sequencer_host_logic():
    from hybrid_linear_memory_amd.layer import PassSequencer, SequenceError
    seq = PassSequencer(n_denoise=2)
    for f in range(3):
        seq.before_read(); seq.after_read()
        seq.before_read(); seq.after_read()
        with pytest.raises(SequenceError):
            seq.before_read()
        seq.before_clean_pass(); seq.after_clean_pass()
        assert seq.frame == f + 1
    with pytest.raises(SequenceError):
        seq.before_clean_pass()          # clean pass before the frame's reads
    seq.restore(7)
    assert seq.frame == 7 and seq.reads == 0
    free = PassSequencer(None)
    free.before_clean_pass(); free.after_clean_pass()
    for _ in range(10):
        free.before_read(); free.after_read()
    with pytest.raises(ValueError):
        PassSequencer(-1)


def test_validation_under_host_sanitizers(tmp_path):
    """The C-ABI layer (csrc/api.cpp) built with g++ under AddressSanitizer and
    UndefinedBehaviorSanitizer, its kernel launchers replaced by host stubs
    (tests/abi_asan/launch_stubs.cpp), and driven through every entry point
    with valid and invalid arguments (tests/abi_asan/abi_check.cpp): every
    status as documented, no sanitizer report."""
    import shutil
    import subprocess
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    here = os.path.join(ROOT, "tests", "abi_asan")
    exe = str(tmp_path / "abi_check")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           os.path.join(ROOT, "hybrid_linear_memory_amd", "csrc", "api.cpp"),
           os.path.join(here, "launch_stubs.cpp"), os.path.join(here, "abi_check.cpp"),
           "-o", exe]
    b = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert b.returncode == 0, b.stdout + b.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "all checks passed" in r.stdout


def test_finiteness_check_host_logic():
    """The layer's debug check (run before any launch) names the first input
    holding a NaN or an infinity and passes finite inputs and None."""
    import torch
    from hybrid_linear_memory_amd.layer import NonFiniteInput, check_finite
    ok = torch.randn(4, 8)
    check_finite(q=ok, k=ok.to(torch.bfloat16), beta=None)
    for bad_value in (float("nan"), float("inf"), float("-inf")):
        bad = ok.clone()
        bad[2, 5] = bad_value
        with pytest.raises(NonFiniteInput, match="^k "):
            check_finite(q=ok, k=bad, v=bad)
        with pytest.raises(NonFiniteInput, match="alpha"):
            check_finite(q=ok, alpha=bad.to(torch.bfloat16))
