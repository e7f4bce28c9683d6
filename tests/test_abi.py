"""The C-ABI library on the CPU: it loads, exports exactly what include/gdr.h
declares, its Python mirror of gdr_shape matches the C layout, and its
synchronous validation rejects bad calls before any launch (every call below
fails validation, so no kernel is ever launched without a GPU)."""
import ctypes
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdr.h")


@pytest.fixture(scope="module")
def gdr():
    import gated_delta_rule_68_amd as g
    if not os.path.exists(g.library_path()):
        from gated_delta_rule_68_amd import build
        build.build(verbose=False)
    g.lib()
    return g


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"GDR_API\s+[\w\s\*]+?\b(gdr_\w+)\s*\(", text)))


def test_header_declares_the_abi():
    assert declared_symbols() == ["gdr_abi_version", "gdr_chunked_fwd",
                                  "gdr_chunked_fwd_gated_rmsnorm", "gdr_chunked_fwd_noalloc",
                                  "gdr_chunked_fwd_split",
                                  "gdr_chunked_path", "gdr_chunked_split_workspace",
                                  "gdr_chunked_workspace_bytes",
                                  "gdr_conv_silu", "gdr_gated_rmsnorm", "gdr_gates",
                                  "gdr_kda_chunked_fwd", "gdr_kda_chunked_fwd_split",
                                  "gdr_kda_chunked_split_workspace", "gdr_kda_chunked_workspace",
                                  "gdr_kda_recurrent_fwd",
                                  "gdr_recurrent_fwd", "gdr_ssd_chunked_fwd",
                                  "gdr_ssd_chunked_fwd_split", "gdr_ssd_chunked_split_workspace",
                                  "gdr_ssd_recurrent_fwd", "gdr_status_string"]


def test_library_exports_every_declared_symbol(gdr):
    lib = gdr.lib()
    for name in declared_symbols():
        assert hasattr(lib, name), f"{name} not exported"
    nm = shutil.which("nm")
    if nm:
        out = subprocess.run([nm, "-D", "--defined-only", gdr.library_path()],
                             capture_output=True, text=True, check=True).stdout
        exported = sorted(set(re.findall(r"\sT\s(gdr_\w+)", out)))
        assert exported == declared_symbols(), "library exports symbols the header does not declare"


def test_abi_version_matches_header(gdr):
    m = re.search(r"#define GDR_ABI_VERSION (\d+)", open(HEADER).read())
    assert gdr.abi_version() == int(m.group(1))


def test_status_strings(gdr):
    lib = gdr.lib()
    seen = set()
    for code in range(8):
        s = lib.gdr_status_string(code).decode()
        assert s and s != "unknown status"
        seen.add(s)
    assert len(seen) == 8
    assert lib.gdr_status_string(99).decode() == "unknown status"


def test_shape_struct_layout_matches_c(gdr, tmp_path):
    """Compile a probe against the header with gcc and compare offsets."""
    gcc = shutil.which("gcc")
    if gcc is None or not os.path.isdir("/opt/rocm/include"):
        pytest.skip("gcc or ROCm headers missing")
    src = tmp_path / "probe.c"
    src.write_text(
        '#include <stdio.h>\n#include <stddef.h>\n#include "gdr.h"\n'
        "int main(void){printf(\"%zu\", sizeof(gdr_shape));"
        + "".join(f'printf(" %zu", offsetof(gdr_shape, {f}));'
                  for f, _ in gdr.GdrShape._fields_) + "return 0;}\n")
    exe = tmp_path / "probe"
    subprocess.run([gcc, "-D__HIP_PLATFORM_AMD__", f"-I{ROOT}/include", "-I/opt/rocm/include",
                    str(src), "-o", str(exe)], check=True, capture_output=True)
    vals = [int(x) for x in subprocess.run([str(exe)], capture_output=True, text=True,
                                           check=True).stdout.split()]
    assert vals[0] == ctypes.sizeof(gdr.GdrShape)
    for (name, _), off in zip(gdr.GdrShape._fields_, vals[1:]):
        assert getattr(gdr.GdrShape, name).offset == off, name


# ------------------------------------------------------------ validation paths
def shape(gdr, **kw):
    s = gdr.GdrShape()
    d = dict(num_seqs=1, seq_len=4, total_tokens=4, cu_seqlens=None, H_k=1, H_v=2, d_k=16,
             d_v=16, dtype=0, chunk=16, scale=0.0, l2_eps=1e-6)
    d.update(kw)
    for k, v in d.items():
        setattr(s, k, v)
    return s


# Fake, never-dereferenced device addresses: every case below fails validation.
BASE = 0x7f0000000000


def fake(i, off=0):
    return ctypes.c_void_p(BASE + i * 0x100000 + off)


def call(gdr, fn, s, ptrs=None):
    p = [fake(i) for i in range(10)] if ptrs is None else ptrs
    f = getattr(gdr.lib(), fn)
    arg = ctypes.byref(s) if s is not None else None
    if fn in ("gdr_kda_chunked_fwd", "gdr_chunked_fwd"):  # no workspace
        return f(arg, *p[:10], None, 0, None)
    return f(arg, *p[:10], None)


@pytest.mark.parametrize("fn", ["gdr_recurrent_fwd", "gdr_chunked_fwd", "gdr_gates"])
def test_null_shape(gdr, fn):
    assert call(gdr, fn, None) == 1


@pytest.mark.parametrize("fn", ["gdr_recurrent_fwd", "gdr_chunked_fwd", "gdr_gates"])
@pytest.mark.parametrize("bad,code", [
    (dict(H_v=3, H_k=2), 2),            # H_v not a multiple of H_k
    (dict(num_seqs=-1), 2),
    (dict(total_tokens=5), 2),          # dense: total != N * T
    (dict(d_k=24), 3),                  # unsupported head size
    (dict(d_v=256), 3),
    (dict(dtype=7), 3),
    (dict(l2_eps=-1.0), 2),
    (dict(scale=float("nan")), 2),
])
def test_shape_errors(gdr, fn, bad, code):
    assert call(gdr, fn, shape(gdr, **bad)) == code


def test_chunk_size_checked(gdr):
    assert call(gdr, "gdr_chunked_fwd", shape(gdr, chunk=48)) == 3
    assert call(gdr, "gdr_chunked_fwd", shape(gdr, chunk=0)) == 3


def test_null_inputs(gdr):
    p = [fake(i) for i in range(10)]
    p[0] = None  # q
    assert call(gdr, "gdr_recurrent_fwd", shape(gdr), p) == 1
    p = [fake(i) for i in range(10)]
    p[5] = None  # A_log
    assert call(gdr, "gdr_chunked_fwd", shape(gdr), p) == 1


def test_misaligned(gdr):
    p = [fake(i) for i in range(10)]
    p[2] = fake(2, off=4)  # v: row tensors need 16 bytes
    assert call(gdr, "gdr_recurrent_fwd", shape(gdr), p) == 4
    p = [fake(i) for i in range(10)]
    p[3] = fake(3, off=2)  # a (fp32): needs 4 bytes
    assert call(gdr, "gdr_recurrent_fwd", shape(gdr), p) == 4


def test_aliasing(gdr):
    p = [fake(i) for i in range(10)]
    p[8] = fake(0)  # o on top of q
    assert call(gdr, "gdr_recurrent_fwd", shape(gdr), p) == 7
    p = [fake(i) for i in range(10)]
    p[9] = fake(7, off=16)  # final_state shifted into initial_state
    assert call(gdr, "gdr_chunked_fwd", shape(gdr), p) == 7


def test_gates_output_alias(gdr):
    p = [fake(i) for i in range(10)]
    p[6] = fake(0)  # q_hat over q
    assert call(gdr, "gdr_gates", shape(gdr), p) == 7


def test_binding_refuses_cpu_tensors(gdr):
    import torch
    q = torch.zeros(4, 1, 16)
    v = torch.zeros(4, 2, 16)
    a = torch.zeros(4, 2)
    with pytest.raises(ValueError):
        gdr.recurrent_fwd(q, q, v, a, a, torch.zeros(2), torch.zeros(2))


def test_chunked_path_selection(gdr):
    lib = gdr.lib()
    assert lib.gdr_chunked_path(ctypes.byref(shape(gdr, dtype=1, d_k=128, d_v=128, chunk=32))) == 1
    assert lib.gdr_chunked_path(ctypes.byref(shape(gdr, dtype=0, d_k=128, d_v=128, chunk=32))) == 2
    assert lib.gdr_chunked_path(ctypes.byref(shape(gdr, dtype=0, d_k=64, d_v=32, chunk=32))) == 2
    assert lib.gdr_chunked_path(ctypes.byref(shape(gdr, dtype=0, d_k=128, d_v=128, chunk=16))) == 0
    assert lib.gdr_chunked_path(ctypes.byref(shape(gdr, dtype=0, d_k=32, d_v=128, chunk=32))) == 0
    assert lib.gdr_chunked_path(ctypes.byref(shape(gdr, dtype=1, d_k=128, d_v=128, chunk=16))) == 0
    assert lib.gdr_chunked_path(ctypes.byref(shape(gdr, dtype=1, d_k=64, d_v=128, chunk=32))) == 0
    assert lib.gdr_chunked_path(ctypes.byref(shape(gdr, dtype=1, d_k=128, d_v=64, chunk=32))) == 1
    assert lib.gdr_chunked_path(ctypes.byref(shape(gdr, dtype=1, d_k=128, d_v=32, chunk=32))) == 0
    assert lib.gdr_chunked_path(ctypes.byref(shape(gdr, chunk=48))) == -3
    assert lib.gdr_chunked_path(ctypes.byref(shape(gdr, H_v=3, H_k=2))) == -2
    assert gdr.chunked_path(16, 48, 128, 128, "bf16", 32) == "matrix_bf16"
    assert gdr.chunked_path(1, 1, 128, 128, "f32", 32) == "matrix_f32"
    assert gdr.chunked_path(1, 1, 128, 128, "f32", 64) == "vector_f32"


# ------------------------------------------ the layer's steps either side of the rule
def conv_call(gdr, s, width=4, **over):
    """gdr_conv_silu with fake pointers; shape(gdr) has C = 2*16 + 2*16 = 64."""
    names = ["x", "weight", "bias", "s_in", "q", "k", "v", "s_out"]
    p = {n: fake(i) for i, n in enumerate(names)}
    p.update(over)
    return gdr.lib().gdr_conv_silu(ctypes.byref(s) if s is not None else None, width,
                                   *[p[n] for n in names], None)


def norm_call(gdr, s, eps=1e-6, **over):
    names = ["o", "z", "weight", "out"]
    p = {n: fake(i) for i, n in enumerate(names)}
    p.update(over)
    return gdr.lib().gdr_gated_rmsnorm(ctypes.byref(s) if s is not None else None, p["o"], p["z"],
                                       p["weight"], eps, p["out"], None)


def test_conv_silu_validation(gdr):
    assert conv_call(gdr, None) == 1                                  # no shape
    assert conv_call(gdr, shape(gdr, H_v=3, H_k=2)) == 2
    assert conv_call(gdr, shape(gdr), width=1) == 3                   # widths 2..4 only
    assert conv_call(gdr, shape(gdr), width=5) == 3
    assert conv_call(gdr, shape(gdr), weight=None) == 1
    assert conv_call(gdr, shape(gdr), x=None) == 1
    assert conv_call(gdr, shape(gdr), v=None) == 1
    assert conv_call(gdr, shape(gdr), x=fake(0, off=8)) == 4          # rows need 16 bytes
    assert conv_call(gdr, shape(gdr), weight=fake(1, off=4)) == 4     # weights move in 16 bytes
    assert conv_call(gdr, shape(gdr), bias=fake(2, off=8)) == 4
    assert conv_call(gdr, shape(gdr, dtype=1), s_in=fake(3, off=1)) == 4
    assert conv_call(gdr, shape(gdr), q=fake(0)) == 7                 # q over x
    assert conv_call(gdr, shape(gdr), k=fake(4, off=64)) == 7         # k inside q
    assert conv_call(gdr, shape(gdr), s_out=fake(3, off=16)) == 7     # shifted over the history


def test_gated_rmsnorm_validation(gdr):
    assert norm_call(gdr, None) == 1
    assert norm_call(gdr, shape(gdr), eps=-1.0) == 2
    assert norm_call(gdr, shape(gdr), eps=float("nan")) == 2
    assert norm_call(gdr, shape(gdr), eps=float("inf")) == 2
    assert norm_call(gdr, shape(gdr), weight=None) == 1
    assert norm_call(gdr, shape(gdr), o=None) == 1
    assert norm_call(gdr, shape(gdr), z=fake(1, off=4)) == 4
    assert norm_call(gdr, shape(gdr), out=fake(0, off=16)) == 7       # shifted over o
    assert norm_call(gdr, shape(gdr), out=fake(2)) == 7               # over the weight
    assert norm_call(gdr, shape(gdr, d_v=24)) == 3


def test_layer_binding_refuses_cpu_tensors(gdr):
    import torch
    x = torch.zeros(4, 64)
    with pytest.raises(ValueError):
        gdr.conv_silu(x, torch.zeros(64, 4), 1, 2, 16, 16)
    o = torch.zeros(4, 2, 16)
    with pytest.raises(ValueError):
        gdr.gated_rmsnorm(o, o, torch.zeros(16))


# ------------------------------------------------------- segmented chunked form
def split_call(gdr, s, seg, ws=None, ws_bytes=1 << 30, **over):
    names = ["q", "k", "v", "a", "b", "A_log", "dt_bias", "s0", "o", "sT"]
    p = {n: fake(i) for i, n in enumerate(names)}
    p.update(over)
    return gdr.lib().gdr_chunked_fwd_split(ctypes.byref(s), seg, *[p[n] for n in names],
                                           fake(20) if ws is None else ws, ws_bytes, None)


def workspace_bytes(gdr, s, seg):
    n = ctypes.c_size_t(0)
    rc = gdr.lib().gdr_chunked_split_workspace(ctypes.byref(s), seg, ctypes.byref(n))
    return rc, n.value


def test_split_workspace_size(gdr):
    # N = 2 sequences of 64 tokens, H_v = 2, d = 16, fp32, chunk 16, segments of 16: P = 4
    s = shape(gdr, num_seqs=2, seq_len=64, total_tokens=128, chunk=16)
    rc, n = workspace_bytes(gdr, s, 16)
    assert rc == 0
    r256 = lambda b: (b + 255) // 256 * 256
    st = 2 * 4 * 2 * 16 * 16 * 4  # N * P * H_v * d_k * d_v * fp32
    assert n == r256(128 * 2 * 16 * 4) + 4 * r256(st)  # zero v, then four state buffers
    assert workspace_bytes(gdr, s, 64) == (0, 0)  # one segment: no workspace


def test_split_workspace_packed_and_wide_values(gdr):
    """A packed batch holds total / segment_len + N segment slots (every
    sequence of L tokens has max(1, ceil(L / segment_len)) segments), plus its
    segment map; d_k != d_v adds the d_k x d_k maps and the M pass's d_k-wide
    outputs."""
    r256 = lambda b: (b + 255) // 256 * 256
    cu = shape(gdr, num_seqs=3, seq_len=0, total_tokens=100, chunk=16)
    cu.cu_seqlens = fake(30).value
    rc, n = workspace_bytes(gdr, cu, 16)
    NP = 100 // 16 + 3
    st = NP * 2 * 16 * 16 * 4
    assert rc == 0
    assert n == r256(100 * 2 * 16 * 4) + 4 * r256(st) + r256((NP + 1) * 4) + r256(4 * 4)
    assert workspace_bytes(gdr, cu, 112) == (0, 0)  # the whole batch fits one segment
    assert workspace_bytes(gdr, cu, 96)[1] > 0
    assert workspace_bytes(gdr, cu, 24)[0] == 2     # not a multiple of the chunk
    # d_k = 32, d_v = 16, dense: M and the identities are d_k x d_k
    s = shape(gdr, num_seqs=2, seq_len=64, total_tokens=128, chunk=16, d_k=32, d_v=16)
    rc, n = workspace_bytes(gdr, s, 16)
    NP = 2 * 4
    st, stm = NP * 2 * 32 * 16 * 4, NP * 2 * 32 * 32 * 4
    assert rc == 0
    assert n == r256(128 * 2 * 32 * 4) + 2 * r256(stm) + 2 * r256(st) + r256(128 * 2 * 32 * 4)


def test_split_validation(gdr):
    s = shape(gdr, num_seqs=1, seq_len=64, total_tokens=64, chunk=16)
    assert split_call(gdr, shape(gdr, num_seqs=1, seq_len=64, total_tokens=64, chunk=16,
                                 d_k=16, d_v=256), 16) == 3   # no kernel for d_v = 256
    cu = shape(gdr, num_seqs=1, seq_len=0, total_tokens=64, chunk=16)
    cu.cu_seqlens = fake(30).value
    assert split_call(gdr, cu, 24) == 2                      # packed: a multiple of the chunk
    assert split_call(gdr, cu, 16, ws_bytes=workspace_bytes(gdr, cu, 16)[1] - 1) == 5
    assert split_call(gdr, s, 0) == 2
    assert split_call(gdr, s, 24) == 2                       # not a multiple of the chunk
    assert split_call(gdr, s, 48) == 2                       # does not divide seq_len
    assert split_call(gdr, s, 16, ws=ctypes.c_void_p(0)) == 1
    _, need = workspace_bytes(gdr, s, 16)
    assert split_call(gdr, s, 16, ws_bytes=need - 1) == 5    # GDR_ERR_WORKSPACE
    assert split_call(gdr, s, 16, ws=fake(20, off=128)) == 4
    assert split_call(gdr, s, 16, ws=fake(8)) == 7           # over o
    assert split_call(gdr, s, 16, o=fake(0)) == 7            # o over q, as gdr_chunked_fwd


def test_ssd_split_validation(gdr):
    """The SSD's segmented form: the SSD's pointer checks, the split's
    segment rules; its workspace equals the rule's for the same shape."""
    lib = gdr.lib()
    names = ["x", "delta", "A", "B", "C", "s0", "z", "y", "sT"]

    def call(s, seg, ws_bytes=1 << 30, **over):
        p = {n: fake(i) for i, n in enumerate(names)}
        p.update(over)
        return lib.gdr_ssd_chunked_fwd_split(ctypes.byref(s), seg, *[p[n] for n in names],
                                             fake(20), ws_bytes, None)
    s = shape(gdr, num_seqs=1, seq_len=64, total_tokens=64, chunk=16)
    assert call(s, 24) == 2                      # not a multiple of the chunk
    assert call(s, 48) == 2                      # does not divide seq_len
    assert call(s, 16, A=None) == 1
    assert call(s, 16, B=fake(3, off=8)) == 4    # rows need 16 bytes
    assert call(s, 16, y=fake(0)) == 7           # y over x
    n_ssd, n_rule = ctypes.c_size_t(0), ctypes.c_size_t(0)
    assert lib.gdr_ssd_chunked_split_workspace(ctypes.byref(s), 16, ctypes.byref(n_ssd)) == 0
    assert lib.gdr_chunked_split_workspace(ctypes.byref(s), 16, ctypes.byref(n_rule)) == 0
    assert n_ssd.value == n_rule.value > 0
    assert call(s, 16, ws_bytes=n_ssd.value - 1) == 5


# ------------------------------------------------------------- the SSD recurrence
SSD_ARGS = ["x", "delta", "A", "B", "C", "s0", "z", "y", "sT"]


def ssd_call(gdr, fn, s, **over):
    p = {n: fake(i) for i, n in enumerate(SSD_ARGS)}
    p.update(over)
    return getattr(gdr.lib(), fn)(ctypes.byref(s) if s is not None else None,
                                  *[p[n] for n in SSD_ARGS], None)


@pytest.mark.parametrize("fn", ["gdr_ssd_recurrent_fwd", "gdr_ssd_chunked_fwd"])
def test_ssd_validation(gdr, fn):
    assert ssd_call(gdr, fn, None) == 1                                  # no shape
    assert ssd_call(gdr, fn, shape(gdr, H_v=3, H_k=2)) == 2              # heads not grouped
    assert ssd_call(gdr, fn, shape(gdr, d_k=24)) == 3                    # state size
    assert ssd_call(gdr, fn, shape(gdr), A=None) == 1
    assert ssd_call(gdr, fn, shape(gdr), C=None) == 1
    assert ssd_call(gdr, fn, shape(gdr), B=fake(3, off=8)) == 4          # rows need 16 bytes
    assert ssd_call(gdr, fn, shape(gdr), A=fake(2, off=2)) == 4
    assert ssd_call(gdr, fn, shape(gdr), y=fake(0)) == 7                 # y over x
    assert ssd_call(gdr, fn, shape(gdr), sT=fake(7)) == 7                # state over y
    assert ssd_call(gdr, fn, shape(gdr), sT=fake(5, off=16)) == 7        # shifted in place


def test_ssd_chunk_checked(gdr):
    assert ssd_call(gdr, "gdr_ssd_chunked_fwd", shape(gdr, chunk=48)) == 3
    assert ssd_call(gdr, "gdr_ssd_chunked_fwd", shape(gdr, chunk=0)) == 3


def test_ssd_binding_refuses_cpu_tensors(gdr):
    import torch
    x = torch.zeros(4, 2, 16)
    with pytest.raises(ValueError):
        gdr.ssd_chunked_fwd(x, torch.zeros(4, 2), torch.zeros(2), torch.zeros(4, 1, 16),
                            torch.zeros(4, 1, 16))


# ------------------------------------------------------- the per-channel decay (KDA)
@pytest.mark.parametrize("fn", ["gdr_kda_recurrent_fwd", "gdr_kda_chunked_fwd"])
def test_kda_validation(gdr, fn):
    assert call(gdr, fn, None) == 1
    assert call(gdr, fn, shape(gdr, H_v=3, H_k=2)) == 2
    assert call(gdr, fn, shape(gdr, d_k=24)) == 3
    p = [fake(i) for i in range(10)]
    p[5] = None  # A_log
    assert call(gdr, fn, shape(gdr), p) == 1
    p = [fake(i) for i in range(10)]
    p[6] = fake(6, off=2)  # dt_bias (fp32)
    assert call(gdr, fn, shape(gdr), p) == 4
    # a holds total x H_v x d_k values here (4 x 2 x 16 fp32 = 512 bytes): an
    # output 64 bytes past its start overlaps it
    p = [fake(i) for i in range(10)]
    p[8] = fake(3, off=64)
    assert call(gdr, fn, shape(gdr), p) == 7
    # ... and so does a final state 64 bytes past the start of dt_bias (2 x 16 fp32)
    p = [fake(i) for i in range(10)]
    p[9] = fake(6, off=64)
    assert call(gdr, fn, shape(gdr), p) == 7


def test_kda_chunk_sizes(gdr):
    assert call(gdr, "gdr_kda_chunked_fwd", shape(gdr, chunk=64)) == 3
    assert call(gdr, "gdr_kda_chunked_fwd", shape(gdr, chunk=48)) == 3


def test_kda_workspace_size(gdr):
    lib = gdr.lib()
    n = ctypes.c_size_t(123)
    # bf16, d_k = 128, chunk 32: one 29,696-byte record per (slot, value head),
    # floor(total / 32) + num_seqs slots
    s = shape(gdr, dtype=1, d_k=128, d_v=64, chunk=32, total_tokens=100, num_seqs=2, seq_len=50)
    assert lib.gdr_kda_chunked_workspace(ctypes.byref(s), ctypes.byref(n)) == 0
    assert n.value == (100 // 32 + 2) * 2 * 29696
    s = shape(gdr, dtype=0, d_k=128, d_v=64, chunk=32)  # fp32: the vector kernel, no workspace
    assert lib.gdr_kda_chunked_workspace(ctypes.byref(s), ctypes.byref(n)) == 0
    assert n.value == 0
    assert lib.gdr_kda_chunked_workspace(ctypes.byref(shape(gdr, chunk=64)), ctypes.byref(n)) == 3
    assert lib.gdr_kda_chunked_workspace(ctypes.byref(s), None) == 1


def test_kda_workspace_checked(gdr):
    f = gdr.lib().gdr_kda_chunked_fwd
    s = shape(gdr, dtype=1, d_k=128, d_v=64, chunk=32)
    need = (4 // 32 + 1) * 2 * 29696
    p = [fake(i) for i in range(10)]
    assert f(ctypes.byref(s), *p, fake(10), need - 1, None) == 5        # too small
    assert f(ctypes.byref(s), *p, fake(10, off=16), need, None) == 4    # not 256-byte aligned
    assert f(ctypes.byref(s), *p, fake(0, off=256), need, None) == 7    # over q
    assert f(ctypes.byref(s), *p, fake(8, off=-4096), need, None) == 7  # runs into o


def test_kda_split_workspace_holds_the_prep(gdr):
    """The KDA split's workspace is the rule's plus, on the two-launch form,
    one prep record per (segment chunk slot, value head)."""
    lib = gdr.lib()
    rule, kda_ = ctypes.c_size_t(0), ctypes.c_size_t(0)
    s = shape(gdr, dtype=1, d_k=128, d_v=128, chunk=32, num_seqs=2, seq_len=1024,
              total_tokens=2048)
    assert lib.gdr_chunked_split_workspace(ctypes.byref(s), 256, ctypes.byref(rule)) == 0
    assert lib.gdr_kda_chunked_split_workspace(ctypes.byref(s), 256, ctypes.byref(kda_)) == 0
    slots = 2048 // 32 + 2 * 4  # 8 segments as sequences
    # the rule's passes run the cooperative form: its workspace for the 8
    # segments as a batch is part of the rule's split workspace, not the KDA's
    seg = shape(gdr, dtype=1, d_k=128, d_v=128, chunk=32, num_seqs=8, seq_len=256,
                total_tokens=2048)
    coop = int(lib.gdr_chunked_workspace_bytes(ctypes.byref(seg)))
    assert coop > 0
    assert kda_.value - (rule.value - (coop + 255) // 256 * 256) >= slots * 2 * 29696
    s = shape(gdr, dtype=0, d_k=128, d_v=128, chunk=32, num_seqs=2, seq_len=1024,
              total_tokens=2048)  # fp32: the vector kernel, no prep
    assert lib.gdr_chunked_split_workspace(ctypes.byref(s), 256, ctypes.byref(rule)) == 0
    assert lib.gdr_kda_chunked_split_workspace(ctypes.byref(s), 256, ctypes.byref(kda_)) == 0
    assert kda_.value == rule.value
    assert lib.gdr_kda_chunked_split_workspace(ctypes.byref(s), 1024, ctypes.byref(kda_)) == 0
    assert kda_.value == 0  # one segment


# ------------------------------------------ the cooperative chunked form's workspace
def chunked_ws_bytes(gdr, **kw):
    return int(gdr.lib().gdr_chunked_workspace_bytes(ctypes.byref(shape(gdr, **kw))))


def test_chunked_workspace_constant_in_sequence_length(gdr):
    """The workspace of gdr_chunked_fwd does not grow with the context: the
    same bytes for 64 and for 32768 tokens (the state is fixed-size,
    GatedDeltaRule.ixx File Reference, "Detailed Description")."""
    def prefill(T):
        return chunked_ws_bytes(gdr, dtype=1, d_k=128, d_v=128, chunk=32, H_k=16, H_v=48,
                                num_seqs=1, seq_len=T, total_tokens=T)
    short, long_ = prefill(64), prefill(32768)
    assert short == long_ > 0
    # a ring of 16 records of 7 KB per value head, and 512 bytes of flags per
    # (sequence, key head) group, after 2 KB of per-XCD counters
    per_head = 16 * 7168
    assert short == 2048 + 16 * (512 + 3 * per_head)
    # packed batches: lengths do not matter either
    s = shape(gdr, dtype=1, d_k=128, d_v=128, chunk=32, H_k=2, H_v=6, num_seqs=3, seq_len=0,
              total_tokens=5000)
    s.cu_seqlens = fake(30).value
    assert int(gdr.lib().gdr_chunked_workspace_bytes(ctypes.byref(s))) == 2048 + 6 * (512 + 3 * per_head)


def test_chunked_workspace_zero_without_cooperative_form(gdr):
    assert chunked_ws_bytes(gdr) == 0                                    # fp32: vector kernel
    assert chunked_ws_bytes(gdr, dtype=1, d_k=128, d_v=128, chunk=16) == 0
    assert chunked_ws_bytes(gdr, dtype=1, d_k=128, d_v=128, chunk=32, H_k=1, H_v=4) == 0  # 4 per key head
    # H_k groups of one sequence that do not fit the device at once: 48 key
    # heads of 3 value heads (16 workgroups a group, 2 groups an XCD)
    assert chunked_ws_bytes(gdr, dtype=1, d_k=128, d_v=128, chunk=32, H_k=48, H_v=144) == 0
    assert int(gdr.lib().gdr_chunked_workspace_bytes(None)) == 0
    assert chunked_ws_bytes(gdr, H_v=3, H_k=2) == 0                      # invalid shape


def test_chunked_workspace_sized_for_one_launch(gdr):
    """A batch with more (sequence, key head) groups than the device holds
    at once runs as consecutive launches on one workspace, sized for the
    sequences one launch holds: 256 sequences of 16 key heads need the
    workspace of one such sequence."""
    one = chunked_ws_bytes(gdr, dtype=1, d_k=128, d_v=128, chunk=32, H_k=16, H_v=48)
    many = chunked_ws_bytes(gdr, dtype=1, d_k=128, d_v=128, chunk=32, H_k=16, H_v=48,
                            num_seqs=256, seq_len=1, total_tokens=256)
    assert many == one == 2048 + 16 * (512 + 3 * 16 * 7168)
    # 2 key heads: 8 sequences (16 groups) a launch
    eight = chunked_ws_bytes(gdr, dtype=1, d_k=128, d_v=128, chunk=32, H_k=2, H_v=6, num_seqs=8,
                             seq_len=4, total_tokens=32)
    assert chunked_ws_bytes(gdr, dtype=1, d_k=128, d_v=128, chunk=32, H_k=2, H_v=6, num_seqs=40,
                            seq_len=4, total_tokens=160) == eight


def test_chunked_workspace_checked(gdr):
    f = gdr.lib().gdr_chunked_fwd
    s = shape(gdr, dtype=1, d_k=128, d_v=128, chunk=32, H_k=1, H_v=3)
    need = int(f and gdr.lib().gdr_chunked_workspace_bytes(ctypes.byref(s)))
    assert need > 0
    p = [fake(i) for i in range(10)]
    assert f(ctypes.byref(s), *p, fake(10), need - 1, None) == 5        # too small
    assert f(ctypes.byref(s), *p, fake(10, off=16), need, None) == 4    # not 256-byte aligned
    assert f(ctypes.byref(s), *p, fake(0, off=256), need, None) == 7    # over q


# ------------------------------------------ the allocation-free chunked entry point
def test_noalloc_validates_like_chunked(gdr):
    fn = "gdr_chunked_fwd_noalloc"
    assert call(gdr, fn, None) == 1
    assert call(gdr, fn, shape(gdr, H_v=3, H_k=2)) == 2
    assert call(gdr, fn, shape(gdr, chunk=48)) == 3
    p = [fake(i) for i in range(10)]
    p[8] = fake(0)  # o on top of q
    assert call(gdr, fn, shape(gdr), p) == 7


def test_noalloc_scratch_limit(gdr):
    """The scratch holds the prefill layer's cooperative workspace (16 key
    heads, 48 value heads, one sequence); a shape that needs more is refused
    with GDR_ERR_WORKSPACE before anything runs."""
    m = re.search(r"#define GDR_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", open(HEADER).read())
    limit = int(m.group(1)) << int(m.group(2))
    assert limit == gdr.NOALLOC_SCRATCH_BYTES
    prefill = dict(dtype=1, d_k=128, d_v=128, chunk=32, H_k=16, H_v=48, num_seqs=1,
                   seq_len=8192, total_tokens=8192)
    assert 0 < chunked_ws_bytes(gdr, **prefill) <= limit
    big = dict(dtype=1, d_k=128, d_v=64, chunk=32, H_k=24, H_v=72, num_seqs=1, seq_len=64,
               total_tokens=64)
    assert chunked_ws_bytes(gdr, **big) > limit
    far = [ctypes.c_void_p(BASE + i * 0x4000000) for i in range(10)]  # 64 MiB apart: no alias
    assert call(gdr, "gdr_chunked_fwd_noalloc", shape(gdr, **big), far) == 5


# ------------------------------------------- chunked form with the norm fused
def call_norm(gdr, s, z=None, w=None, eps=1e-6, out=None, ws=None, ws_bytes=0, ptrs=None):
    """gdr_chunked_fwd_gated_rmsnorm with fake pointers: q..dt_bias, s0 from
    slots 0..7, z slot 10, weight slot 11, out slot 8, final state slot 9."""
    p = [fake(i) for i in range(12)] if ptrs is None else ptrs
    f = gdr.lib().gdr_chunked_fwd_gated_rmsnorm
    arg = ctypes.byref(s) if s is not None else None
    return f(arg, *p[:8], p[10] if z is None else z, p[11] if w is None else w,
             ctypes.c_float(eps), p[8] if out is None else out, p[9], ws, ctypes.c_size_t(ws_bytes),
             None)


def test_norm_fused_null_shape(gdr):
    assert call_norm(gdr, None) == 1


@pytest.mark.parametrize("eps", [-1.0, float("nan"), float("inf")])
def test_norm_fused_bad_eps(gdr, eps):
    assert call_norm(gdr, shape(gdr), eps=eps) == 2


def test_norm_fused_null_weight_and_z(gdr):
    assert call_norm(gdr, shape(gdr), w=ctypes.c_void_p(0)) == 1
    assert call_norm(gdr, shape(gdr), z=ctypes.c_void_p(0)) == 1


def test_norm_fused_alignment(gdr):
    assert call_norm(gdr, shape(gdr), z=fake(10, 8)) == 4       # z rows move in 16-byte vectors
    assert call_norm(gdr, shape(gdr), w=fake(11, 2)) == 4       # fp32 weight


def test_norm_fused_alias(gdr):
    # z (4 tokens x 2 heads x 16 fp32 = 512 bytes) overlapping out, exactly or shifted
    assert call_norm(gdr, shape(gdr), z=fake(8)) == 7
    assert call_norm(gdr, shape(gdr), z=fake(8, 256)) == 7
    # the weight inside the final state
    assert call_norm(gdr, shape(gdr), w=fake(9, 64)) == 7


def test_norm_fused_shape_errors_come_first(gdr):
    assert call_norm(gdr, shape(gdr, H_v=3, H_k=2)) == 2
    assert call_norm(gdr, shape(gdr, chunk=8)) == 3
