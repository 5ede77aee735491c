"""The C ABI on the host: the library loads without a GPU, exports every
function include/parallax.h declares, and rejects each invalid argument with
its status code before any HIP call (fake, never-dereferenced pointers)."""
import ctypes
import os
import re

import pytest

import parallax_local_linear_decode_amd as plx

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include",
                      "parallax.h")
FAKE = 0x7F0000000000  # 16-byte aligned, never dereferenced


@pytest.fixture(scope="module")
def lib():
    return plx.load_library()


def test_exports_every_declared_function(lib):
    text = open(HEADER).read()
    names = set(re.findall(r"\b(parallax_[a-z_]+)\s*\(", text))
    assert {"parallax_decode", "parallax_prefill", "parallax_decode_workspace_size",
            "parallax_decode_no_alloc",
            "parallax_prefill_backward", "parallax_prefill_backward_workspace_size",
            "parallax_decode_lla", "parallax_decode_lla_workspace_size", "parallax_qr_projection",
            "parallax_status_string", "parallax_last_error", "parallax_abi_version"} <= names
    for n in sorted(names):
        assert hasattr(lib, n), f"{n} is declared but not exported"


def test_abi_version_and_strings(lib):
    assert lib.parallax_abi_version() == plx.ABI_VERSION
    for code, name in [(0, "PARALLAX_OK"), (1, "PARALLAX_ERR_INVALID_ARG"),
                       (2, "PARALLAX_ERR_UNSUPPORTED"), (3, "PARALLAX_ERR_WORKSPACE"),
                       (4, "PARALLAX_ERR_HIP")]:
        assert plx.parallax_status_string(code) == name


def good_decode(**over):
    a = plx.DecodeArgs()
    a.struct_size = ctypes.sizeof(plx.DecodeArgs)
    a.batch, a.num_q_heads, a.num_kv_heads, a.head_dim = 8, 16, 8, 128
    a.scale = 128 ** -0.5
    a.q = a.rho = a.out = a.k = a.v = FAKE
    a.q_stride_b, a.q_stride_h = 16 * 128, 128
    a.rho_stride_b, a.rho_stride_h = 16 * 128, 128
    a.out_stride_b, a.out_stride_h = 16 * 128, 128
    a.kv_dtype = plx.PARALLAX_BF16
    a.k_stride_0, a.k_stride_h, a.k_stride_t = 8 * 4096 * 128, 4096 * 128, 128
    a.v_stride_0, a.v_stride_h, a.v_stride_t = 8 * 4096 * 128, 4096 * 128, 128
    a.max_seq_len = 4096
    for k, v in over.items():
        setattr(a, k, v)
    return a


def ws_size(lib, a):
    n = ctypes.c_size_t(123)
    st = lib.parallax_decode_workspace_size(ctypes.byref(a), ctypes.byref(n))
    return st, n.value


def test_valid_decode_plan(lib):
    st, n = ws_size(lib, good_decode())
    assert st == plx.PARALLAX_OK and n > 0
    # a single split needs no workspace
    st, n = ws_size(lib, good_decode(split_tokens=4096))
    assert st == plx.PARALLAX_OK and n == 0
    # explicit split: one record (A, B: d floats each; m, Z, R, pad) per split and head,
    # then one 8-byte arrival flag per split for the in-kernel merge
    st, n = ws_size(lib, good_decode(split_tokens=1024))
    assert n == 64 * 4 * 2 * (2 * 128 + 4) * 4 + 64 * 4 * 8


INVALID = plx.PARALLAX_ERR_INVALID_ARG
UNSUPP = plx.PARALLAX_ERR_UNSUPPORTED


@pytest.mark.parametrize("over,status,needle", [
    (dict(struct_size=8), INVALID, "struct_size"),
    (dict(batch=0), INVALID, "batch"),
    (dict(num_kv_heads=3), INVALID, "num_q_heads"),
    (dict(num_q_heads=24), UNSUPP, "group"),
    (dict(head_dim=96), UNSUPP, "head_dim"),
    (dict(kv_dtype=7), INVALID, "kv_dtype"),
    (dict(scale=float("nan")), INVALID, "scale"),
    (dict(q=None), INVALID, "non-NULL"),
    (dict(v=None), INVALID, "non-NULL"),
    (dict(max_seq_len=0), INVALID, "max_seq_len"),
    (dict(k_stride_t=-128), INVALID, "non-negative"),
    (dict(k=FAKE + 4), UNSUPP, "aligned"),
    (dict(out=FAKE + 8), UNSUPP, "aligned"),
    (dict(k_stride_t=132), UNSUPP, "16 bytes"),
    (dict(q_stride_h=130), UNSUPP, "16 bytes"),
    (dict(split_tokens=100), INVALID, "split_tokens"),
    (dict(split_tokens=64), INVALID, "split_tokens"),
    (dict(split_tokens=-256), INVALID, "split_tokens"),
    (dict(window=-1), INVALID, "window"),
    (dict(block_table=FAKE, block_size=16, max_blocks_per_seq=256), INVALID, "seq_lens"),
    (dict(block_table=FAKE, seq_lens=FAKE, block_size=32, max_blocks_per_seq=256), UNSUPP,
     "block_size"),
    (dict(block_table=FAKE, seq_lens=FAKE, block_size=16, max_blocks_per_seq=100), INVALID,
     "max_blocks_per_seq"),
    (dict(block_table=FAKE, seq_lens=FAKE, block_size=16, max_blocks_per_seq=0), INVALID,
     "max_blocks_per_seq"),
])
def test_decode_rejects(lib, over, status, needle):
    a = good_decode(**over)
    st, _ = ws_size(lib, a)
    assert st == status
    assert needle in plx.parallax_last_error()
    st = lib.parallax_decode(ctypes.byref(a), FAKE, 1 << 30, None)
    assert st == status
    # the no-allocation variant runs the same checks, also before any HIP call
    assert lib.parallax_decode_no_alloc(ctypes.byref(a), None) == status
    assert needle in plx.parallax_last_error()


def test_decode_no_alloc_rejects_an_explicit_split_beyond_its_scratch(lib):
    """2048 sequences x 8 KV heads x 2 query heads in 256-token splits of
    32768 tokens: 128 splits of 1040-byte records per head are 4.4 GB, far
    beyond the library's scratch, so an explicit split is refused (on the
    host, before any HIP call)."""
    a = good_decode(batch=2048, max_seq_len=32768, split_tokens=256,
                    k_stride_0=8 * 32768 * 128, k_stride_h=32768 * 128,
                    v_stride_0=8 * 32768 * 128, v_stride_h=32768 * 128)
    st, need = ws_size(lib, a)
    assert st == 0 and need > plx.NO_ALLOC_SCRATCH_BYTES
    assert lib.parallax_decode_no_alloc(ctypes.byref(a), None) == plx.PARALLAX_ERR_WORKSPACE
    assert "scratch" in plx.parallax_last_error()
    assert lib.parallax_decode_no_alloc(None, None) == INVALID


def test_decode_null_args(lib):
    assert lib.parallax_decode(None, None, 0, None) == INVALID
    n = ctypes.c_size_t(0)
    assert lib.parallax_decode_workspace_size(None, ctypes.byref(n)) == INVALID
    assert lib.parallax_decode_workspace_size(ctypes.byref(good_decode()), None) == INVALID


def test_decode_workspace_checks(lib):
    a = good_decode()
    st, need = ws_size(lib, a)
    assert need > 0
    assert lib.parallax_decode(ctypes.byref(a), None, need, None) == plx.PARALLAX_ERR_WORKSPACE
    assert lib.parallax_decode(ctypes.byref(a), FAKE, need - 1, None) == \
        plx.PARALLAX_ERR_WORKSPACE
    assert lib.parallax_decode(ctypes.byref(a), FAKE + 4, need, None) == \
        plx.PARALLAX_ERR_WORKSPACE
    assert "workspace" in plx.parallax_last_error()


def good_prefill(**over):
    a = plx.PrefillArgs()
    a.struct_size = ctypes.sizeof(plx.PrefillArgs)
    a.batch, a.seq_len, a.num_q_heads, a.num_kv_heads, a.head_dim = 4, 8192, 16, 8, 128
    a.scale = 128 ** -0.5
    a.causal = 1
    a.q = a.rho = a.k = a.v = a.out = FAKE
    a.q_stride_b, a.q_stride_s, a.q_stride_h = 8192 * 16 * 128, 16 * 128, 128
    a.rho_stride_b, a.rho_stride_s, a.rho_stride_h = 8192 * 16 * 128, 16 * 128, 128
    a.k_stride_b, a.k_stride_s, a.k_stride_h = 8192 * 8 * 128, 8 * 128, 128
    a.v_stride_b, a.v_stride_s, a.v_stride_h = 8192 * 8 * 128, 8 * 128, 128
    a.out_stride_b, a.out_stride_s, a.out_stride_h = 8192 * 16 * 128, 16 * 128, 128
    for k, v in over.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("over,status,needle", [
    (dict(struct_size=4), INVALID, "struct_size"),
    (dict(seq_len=0), INVALID, "seq_len"),
    (dict(num_kv_heads=5), INVALID, "num_q_heads"),
    (dict(scale=float("inf")), INVALID, "scale"),
    (dict(rho=None), INVALID, "non-NULL"),
    (dict(k_stride_s=-1), INVALID, "non-negative"),
    (dict(causal=0), UNSUPP, "causal"),
    (dict(head_dim=96), UNSUPP, "head_dim"),
    (dict(num_q_heads=256), UNSUPP, "GQA group"),
    (dict(num_q_heads=24), UNSUPP, "GQA group"),
    (dict(v=FAKE + 2), UNSUPP, "aligned"),
    (dict(q_stride_s=2052), UNSUPP, "16 bytes"),
    (dict(out_stride_h=130), UNSUPP, "16 bytes"),
    (dict(window=-5), INVALID, "window"),
    (dict(workgroups=-1), INVALID, "workgroups"),
])
def test_prefill_rejects(lib, over, status, needle):
    a = good_prefill(**over)
    assert lib.parallax_prefill(ctypes.byref(a), None) == status
    assert needle in plx.parallax_last_error()
    assert lib.parallax_prefill(None, None) == INVALID


def test_older_structs_are_rejected(lib):
    """ABI version 2 appended `window` to both argument structs, version 3
    the three optional statistics outputs to the prefill struct and version 5
    its `workgroups`; a caller built against an older header passes a
    smaller struct_size."""
    old_decode = ctypes.sizeof(plx.DecodeArgs) - 8
    st, _ = ws_size(lib, good_decode(struct_size=old_decode))
    assert st == INVALID and "struct_size" in plx.parallax_last_error()
    v5 = ctypes.sizeof(plx.PrefillArgs)
    assert plx.PrefillArgs.workgroups.offset + 4 <= v5 and plx.PrefillArgs.o_sa.offset + 8 <= v5
    for old_prefill in (plx.PrefillArgs.workgroups.offset, plx.PrefillArgs.lse.offset,
                        plx.PrefillArgs.lse.offset - 8):
        a = good_prefill(struct_size=old_prefill)
        assert lib.parallax_prefill(ctypes.byref(a), None) == INVALID
        assert "struct_size" in plx.parallax_last_error()


def test_prefill_stats_outputs_must_be_aligned(lib):
    for name in ("lse", "rmean", "o_sa"):
        a = good_prefill(**{name: FAKE + 4})
        assert lib.parallax_prefill(ctypes.byref(a), None) == UNSUPP
        assert "aligned" in plx.parallax_last_error()


def good_backward(**over):
    a = plx.PrefillBackwardArgs()
    a.struct_size = ctypes.sizeof(plx.PrefillBackwardArgs)
    a.batch, a.seq_len, a.num_q_heads, a.num_kv_heads, a.head_dim = 4, 8192, 16, 8, 128
    a.scale = 128 ** -0.5
    a.causal = 1
    for n in ("q", "rho", "k", "v", "dout", "out", "o_sa", "lse", "rmean", "dq", "drho", "dk",
              "dv"):
        setattr(a, n, FAKE)
    qs = (8192 * 16 * 128, 16 * 128, 128)
    ks = (8192 * 8 * 128, 8 * 128, 128)
    for pre, st in (("q", qs), ("rho", qs), ("dout", qs), ("out", qs), ("dq", qs), ("k", ks),
                    ("v", ks), ("dk", ks)):
        setattr(a, pre + "_stride_b", st[0])
        setattr(a, pre + "_stride_s", st[1])
        setattr(a, pre + "_stride_h", st[2])
    for k, v in over.items():
        setattr(a, k, v)
    return a


def bw_size(lib, a):
    n = ctypes.c_size_t(123)
    st = lib.parallax_prefill_backward_workspace_size(ctypes.byref(a), ctypes.byref(n))
    return st, n.value


def test_backward_workspace_size(lib):
    """One float4 of row statistics per (batch, query head, row)."""
    assert bw_size(lib, good_backward()) == (plx.PARALLAX_OK, 4 * 16 * 8192 * 16)
    assert bw_size(lib, good_backward(seq_len=5, batch=1)) == (plx.PARALLAX_OK, 16 * 5 * 16)
    assert lib.parallax_prefill_backward_workspace_size(ctypes.byref(good_backward()), None) == \
        INVALID


@pytest.mark.parametrize("over,status,needle", [
    (dict(struct_size=8), INVALID, "struct_size"),
    (dict(batch=0), INVALID, "batch"),
    (dict(num_kv_heads=3), INVALID, "num_q_heads"),
    (dict(scale=float("nan")), INVALID, "scale"),
    (dict(dout=None), INVALID, "non-NULL"),
    (dict(lse=None), INVALID, "non-NULL"),
    (dict(dv=None), INVALID, "non-NULL"),
    (dict(dk_stride_s=-4), INVALID, "non-negative"),
    (dict(window=-1), INVALID, "window"),
    (dict(causal=0), UNSUPP, "causal"),
    (dict(head_dim=96), UNSUPP, "head_dim"),
    (dict(num_q_heads=256), UNSUPP, "GQA group"),
    (dict(rmean=FAKE + 8), UNSUPP, "aligned"),
    (dict(dout_stride_h=132), UNSUPP, "16 bytes"),
    (dict(dq_stride_s=2050), UNSUPP, "16 bytes"),
])
def test_backward_rejects(lib, over, status, needle):
    a = good_backward(**over)
    assert bw_size(lib, a)[0] == status
    assert needle in plx.parallax_last_error()
    assert lib.parallax_prefill_backward(ctypes.byref(a), FAKE, 1 << 30, None) == status
    assert lib.parallax_prefill_backward(None, FAKE, 1 << 30, None) == INVALID


def test_backward_workspace_checks(lib):
    a = good_backward()
    _, need = bw_size(lib, a)
    assert lib.parallax_prefill_backward(ctypes.byref(a), None, need, None) == \
        plx.PARALLAX_ERR_WORKSPACE
    assert lib.parallax_prefill_backward(ctypes.byref(a), FAKE, need - 16, None) == \
        plx.PARALLAX_ERR_WORKSPACE
    assert lib.parallax_prefill_backward(ctypes.byref(a), FAKE + 8, need, None) == \
        plx.PARALLAX_ERR_WORKSPACE
    assert "workspace" in plx.parallax_last_error()


def test_window_shrinks_the_split_plan(lib):
    """A local window bounds the tokens a row's splits cover (window + 31), so
    fewer splits and less workspace than full attention over the cache."""
    full = good_decode(batch=1, max_seq_len=32768,
                       k_stride_0=8 * 32768 * 128, k_stride_h=32768 * 128,
                       v_stride_0=8 * 32768 * 128, v_stride_h=32768 * 128)
    st, n_full = ws_size(lib, full)
    assert st == plx.PARALLAX_OK and n_full > 0
    full.window = 100
    st, n_win = ws_size(lib, full)
    assert st == plx.PARALLAX_OK and n_win == 0
    full.window = 40000  # at least the cache: same plan as full attention
    assert ws_size(lib, full) == (plx.PARALLAX_OK, n_full)


def good_lla(**over):
    la = plx.LlaArgs()
    la.struct_size = ctypes.sizeof(plx.LlaArgs)
    la.lam, la.iterations = 0.5, 16
    la.rho_out = la.resid = FAKE
    for k, v in over.items():
        setattr(la, k, v)
    return la


def lla_size(lib, a, la):
    n = ctypes.c_size_t(7)
    st = lib.parallax_decode_lla_workspace_size(ctypes.byref(a), ctypes.byref(la), ctypes.byref(n))
    return st, n.value


def test_lla_workspace_size(lib):
    """The decode partials (rounded up to 256 bytes), then five [B, Hq, d]
    conjugate-gradient vectors and two squared norms per row; rho is not
    read, so it may be NULL."""
    a = good_decode(rho=None)
    st, dec = ws_size(lib, good_decode())
    assert st == plx.PARALLAX_OK
    st, n = lla_size(lib, a, good_lla())
    assert st == plx.PARALLAX_OK
    assert n == (dec + 255) // 256 * 256 + (5 * 8 * 16 * 128 + 2 * 8 * 16) * 4


@pytest.mark.parametrize("over,status,needle", [
    (dict(struct_size=16), INVALID, "struct_size"),
    (dict(lam=0.0), INVALID, "lambda"),
    (dict(lam=-1.0), INVALID, "lambda"),
    (dict(lam=float("nan")), INVALID, "lambda"),
    (dict(iterations=0), INVALID, "iterations"),
    (dict(iterations=5000), INVALID, "iterations"),
    (dict(rho_out=FAKE + 4), UNSUPP, "aligned"),
])
def test_lla_rejects(lib, over, status, needle):
    a = good_decode(rho=None)
    la = good_lla(**over)
    assert lla_size(lib, a, la)[0] == status
    assert needle in plx.parallax_last_error()
    assert lib.parallax_decode_lla(ctypes.byref(a), ctypes.byref(la), FAKE, 1 << 30, None) == status


def test_lla_checks_the_decode_arguments(lib):
    la = good_lla()
    assert lla_size(lib, good_decode(num_kv_heads=3), la)[0] == INVALID
    assert lla_size(lib, good_decode(head_dim=96), la)[0] == UNSUPP
    assert lla_size(lib, good_decode(struct_size=8), la)[0] == INVALID
    assert "struct_size" in plx.parallax_last_error()
    assert lib.parallax_decode_lla(None, ctypes.byref(la), FAKE, 1 << 30, None) == INVALID
    assert lib.parallax_decode_lla(ctypes.byref(good_decode()), None, FAKE, 1 << 30, None) == \
        INVALID


def test_lla_workspace_checks(lib):
    a, la = good_decode(rho=None), good_lla()
    _, need = lla_size(lib, a, la)
    assert lib.parallax_decode_lla(ctypes.byref(a), ctypes.byref(la), FAKE, need - 4, None) == \
        plx.PARALLAX_ERR_WORKSPACE
    assert lib.parallax_decode_lla(ctypes.byref(a), ctypes.byref(la), None, need, None) == \
        plx.PARALLAX_ERR_WORKSPACE
    assert lib.parallax_decode_lla(ctypes.byref(a), ctypes.byref(la), FAKE + 8, need, None) == \
        plx.PARALLAX_ERR_WORKSPACE


def good_projection(**over):
    a = plx.ProjectionArgs()
    a.struct_size = ctypes.sizeof(plx.ProjectionArgs)
    a.tokens, a.model_dim, a.num_q_heads, a.head_dim = 8, 2048, 16, 128
    a.out_dtype = plx.PARALLAX_F32
    a.x = a.w_q = a.w_r = a.q = a.rho = FAKE
    a.x_stride_t, a.w_stride_n = 2048, 2048
    a.q_stride_t, a.q_stride_h = 2048, 128
    a.rho_stride_t, a.rho_stride_h = 2048, 128
    for k, v in over.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("over,status,needle", [
    (dict(struct_size=12), INVALID, "struct_size"),
    (dict(tokens=0), INVALID, "tokens"),
    (dict(out_dtype=7), INVALID, "out_dtype"),
    (dict(w_r=None), INVALID, "non-NULL"),
    (dict(q_stride_h=-128), INVALID, "non-negative"),
    (dict(model_dim=2176), UNSUPP, "multiple of 256"),
    (dict(head_dim=96), UNSUPP, "head_dim"),
    (dict(x=FAKE + 2), UNSUPP, "aligned"),
    (dict(x_stride_t=2052), UNSUPP, "16 bytes"),
    (dict(out_dtype=plx.PARALLAX_BF16, q_stride_h=132), UNSUPP, "16 bytes"),
    (dict(tokens=(1 << 22) + 1), UNSUPP, "tokens"),
])
def test_projection_rejects(lib, over, status, needle):
    a = good_projection(**over)
    assert lib.parallax_qr_projection(ctypes.byref(a), None) == status
    assert needle in plx.parallax_last_error()
    assert lib.parallax_qr_projection(None, None) == INVALID


def test_probe_library_exports_its_kernels_and_rejects_bad_arguments():
    """The benchmark's reference kernels (read stream, decode-shaped read,
    matrix/vector issue probe) live in their own library; its launchers check
    their arguments on the host before any HIP call."""
    path = os.path.join(os.path.dirname(plx.LIB_PATH), "libparallax_probe.so")
    probe = ctypes.CDLL(path)
    for n in ("parallax_probe_read", "parallax_probe_read_decode_shape", "parallax_probe_issue"):
        assert hasattr(probe, n), n
    probe.parallax_probe_issue.argtypes = [ctypes.c_int] * 4 + [ctypes.c_void_p] * 2
    probe.parallax_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                          ctypes.c_void_p]
    assert probe.parallax_probe_issue(16, 1, 1, 256, FAKE, None) == 1   # unknown mode bit
    assert probe.parallax_probe_issue(1, -1, 1, 256, FAKE, None) == 1   # negative count
    assert probe.parallax_probe_issue(1, 1, 1, 0, FAKE, None) == 1      # no workgroups
    assert probe.parallax_probe_issue(1, 1, 1, 256, None, None) == 1    # no sink
    assert probe.parallax_probe_read(FAKE, 24, FAKE, None) == 1         # not whole 16 bytes
