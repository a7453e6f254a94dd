"""Host-side checks of the C ABI (no GPU needed, no kernel is launched).

Every function declared in include/gdn2.h must be exported by libgdn2.so, and
argument checks must reject bad calls before any launch (fake, never
dereferenced pointers are used where a check is expected to fail first)."""
import ctypes
import os
import re

import pytest

import linear_attention_sequence_gdn2_amd as gdn2

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn2.h")
OK, INVALID, UNSUPPORTED, WORKSPACE = 0, 1, 2, 3
P = ctypes.c_void_p


def _library_cus():
    """The compute-unit count the library sizes its launches from: the device's, or 256 when
    no device answers (a host without a GPU)."""
    import torch
    if not torch.cuda.is_available():
        return 256
    return torch.cuda.get_device_properties(0).multi_processor_count


# launch-shape and workspace expectations computed for 256 compute units (an MI355X, or a host
# with no device); on a device partitioned into fewer CUs the library picks other launches
cus_256 = pytest.mark.skipif(_library_cus() != 256, reason="expectations assume 256 compute units")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn2_[a-z_0-9]+)\s*\(", text)))


def test_library_is_built():
    assert os.path.exists(gdn2.LIB_PATH), "run python -m linear_attention_sequence_gdn2_amd.build"


def test_every_declared_symbol_is_exported():
    lib = gdn2.load()
    names = _declared()
    assert len(names) >= 10, names
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, missing
    assert sorted(names) == sorted(gdn2.EXPORTS)


def _shape(B=2, T=100, H=3, dk=128, dv=64, chunk=64, dt=1, gates=0, scalar=0):
    return gdn2.Gdn2Shape(B, T, H, dk, dv, chunk, dt, gates, scalar)


def test_shape_struct_matches_header():
    text = open(HEADER).read()
    body = re.search(r"typedef struct \{(.*?)\} gdn2_shape;", text, flags=re.S).group(1)
    body = re.sub(r"/\*.*?\*/", "", body, flags=re.S)
    fields = [f.strip() for decl in body.split(";") if decl.strip()
              for f in decl.strip()[len("int "):].split(",")]
    assert fields == [f[0] for f in gdn2.Gdn2Shape._fields_]
    assert ctypes.sizeof(gdn2.Gdn2Shape) == 4 * len(fields)


def _flags(items):
    # one strong-decay flag (int) per chunk after the records, rounded up to 256 bytes
    return (items * 4 + 255) // 256 * 256


# per chunk: the chunk operand record (Kh, Et, Qt rows and T split in bf16, 16 P^T and 16 P
# fragment tiles, the decay scan's offsets per token block and channel, gamma; rounded up to 256)
RECORD = (6 * 64 * 128 * 2 + 2 * 64 * 64 * 2 + 2 * 16 * 64 * 16 + 4 * 128 * 4 + 128 * 4 + 255) // 256 * 256


@cus_256
def test_workspace_and_state_sizes():
    lib = gdn2.load()
    s = _shape()
    nc = (100 + 63) // 64
    one = 2 * 3 * nc * 128 * 64 * 4
    assert lib.gdn2_chunk_states_bytes(ctypes.byref(s)) == one
    # per chunk: the adjoint factors R, Q2^T, then the chunk operand records, then the flags
    items = 2 * 3 * nc
    factors = items * ((128 * 128 + 64 * 128) * 4 + RECORD) + _flags(items)
    assert lib.gdn2_chunk_factors_bytes(ctypes.byref(s)) == factors
    assert lib.gdn2_chunk_bwd_workspace_size(ctypes.byref(s)) == 2 * one + factors
    # forward-only records and their flags
    assert lib.gdn2_chunk_fwd_workspace_size(ctypes.byref(s)) == items * RECORD + _flags(items)
    bad = _shape(dk=96)
    assert lib.gdn2_chunk_states_bytes(ctypes.byref(bad)) == ctypes.c_size_t(-1).value
    # the widest rows accepted: H * max(dk, dv) just under 2^24
    wide = _shape(B=1, T=64, H=(1 << 17) - 1, dk=128, dv=128)
    assert lib.gdn2_chunk_states_bytes(ctypes.byref(wide)) == ((1 << 17) - 1) * 128 * 128 * 4


@pytest.mark.parametrize("kw,code", [
    (dict(B=0), INVALID), (dict(T=0), INVALID), (dict(H=-1), INVALID),
    (dict(chunk=32), UNSUPPORTED), (dict(dk=96), UNSUPPORTED), (dict(dv=256), UNSUPPORTED),
    (dict(dt=7), UNSUPPORTED), (dict(B=1 << 14, T=1 << 14, H=16), UNSUPPORTED),
    (dict(B=1, T=64, H=1 << 17, dk=128, dv=128), UNSUPPORTED),   # 64 rows of H*d fp32 span 4 GiB
    (dict(B=1, T=64, H=1 << 18, dk=64, dv=32), UNSUPPORTED),
    (dict(gates=2), UNSUPPORTED), (dict(gates=1, dt=0), UNSUPPORTED),
    (dict(scalar=8), UNSUPPORTED), (dict(scalar=1, dt=0), UNSUPPORTED), (dict(scalar=6, gates=1), UNSUPPORTED),
])
def test_shape_checks(kw, code):
    lib = gdn2.load()
    s = _shape(**kw)
    fake = P(0x10000)
    rc = lib.gdn2_chunk_fwd(ctypes.byref(s), fake, fake, fake, fake, fake, fake, None, fake, None, None, 0, None)
    assert rc == code


def test_null_shape_and_pointers():
    lib = gdn2.load()
    fake = P(0x10000)
    assert lib.gdn2_chunk_fwd(None, fake, fake, fake, fake, fake, fake, None, fake, None, None, 0, None) == INVALID
    s = _shape()
    for i in range(7):
        args = [fake] * 6 + [None, fake, None]
        idx = [0, 1, 2, 3, 4, 5, 7][i]
        args[idx] = None
        assert lib.gdn2_chunk_fwd(ctypes.byref(s), *args, None, 0, None) == INVALID


def test_misaligned_pointer_rejected():
    lib = gdn2.load()
    s = _shape()
    fake, odd = P(0x10000), P(0x10008)
    assert lib.gdn2_chunk_fwd(ctypes.byref(s), fake, odd, fake, fake, fake, fake, None, fake, None, None, 0,
                              None) == INVALID


def test_per_token_gates_need_only_word_alignment():
    """A per-token gate may sit at any 4-byte address; the others still need 16 bytes."""
    lib = gdn2.load()
    f, word, odd = P(0x10000), P(0x10004), P(0x10002)
    s = _shape(scalar=1)   # log_alpha per token
    # a gate that is not per token and is only word-aligned is rejected before any launch
    assert lib.gdn2_chunk_fwd(ctypes.byref(s), f, f, f, f, word, f, None, f, None, None, 0, None) == INVALID
    assert lib.gdn2_chunk_fwd(ctypes.byref(s), f, f, f, odd, f, f, None, f, None, None, 0, None) == INVALID
    g = [f] * 6 + [f] * 3 + [f] * 3
    g[9] = odd   # dlog_alpha per token, not word aligned
    assert lib.gdn2_chunk_bwd_grads(ctypes.byref(s), *g[:6], *g[6:9], f, f, f, f, *g[9:], None) == INVALID
    s = _shape(T=1, scalar=4)   # w per token in a step; b misaligned
    assert lib.gdn2_step(ctypes.byref(s), f, f, f, f, word, word, None, f, f, None) == INVALID


def test_backward_workspace_checked_before_launch():
    lib = gdn2.load()
    s = _shape()
    f = P(0x10000)
    need = lib.gdn2_chunk_bwd_workspace_size(ctypes.byref(s))
    args = [f] * 6 + [None, f, None] + [f] * 6 + [None]
    assert lib.gdn2_chunk_bwd(ctypes.byref(s), *args, None, need, None) == WORKSPACE
    assert lib.gdn2_chunk_bwd(ctypes.byref(s), *args, f, need - 1, None) == WORKSPACE


def test_staged_entry_points_check_arguments():
    lib = gdn2.load()
    s = _shape()
    f = P(0x10000)
    assert lib.gdn2_chunk_bwd_factors(ctypes.byref(s), f, f, f, f, None, None) == INVALID
    assert lib.gdn2_chunk_bwd_factors(ctypes.byref(s), f, f, f, P(0x10008), f, None) == INVALID
    assert lib.gdn2_chunk_bwd_reverse(ctypes.byref(s), f, f, None, None, None, None) == INVALID
    assert lib.gdn2_chunk_bwd_reverse(ctypes.byref(s), None, f, None, f, None, None) == INVALID
    assert lib.gdn2_chunk_bwd_grads(ctypes.byref(s), f, f, f, f, f, f, f, f, f, f, f, f, f, f, f, None, None) == INVALID
    # the factor buffer is required and checked before any launch
    assert lib.gdn2_chunk_bwd_grads(ctypes.byref(s), f, f, f, f, f, f, f, f, f, None, f, f, f, f, f, f, None) == INVALID
    assert lib.gdn2_chunk_bwd_grads(ctypes.byref(s), f, f, f, f, f, f, f, f, f, P(0x10008), f, f, f, f, f, f,
                                    None) == INVALID


def test_step_checks_arguments():
    lib = gdn2.load()
    f = P(0x10000)
    s = _shape(T=2)
    assert lib.gdn2_step(ctypes.byref(s), f, f, f, f, f, f, None, f, f, None) == INVALID   # T must be 1
    s = _shape(T=1)
    assert lib.gdn2_step(ctypes.byref(s), f, f, f, f, f, f, None, None, f, None) == INVALID
    assert lib.gdn2_step(ctypes.byref(s), f, f, f, f, f, P(0x10004), None, f, f, None) == INVALID
    s = _shape(T=1, dk=96)
    assert lib.gdn2_step(ctypes.byref(s), f, f, f, f, f, f, None, f, f, None) == UNSUPPORTED


def test_strerror_covers_every_status():
    lib = gdn2.load()
    msgs = {lib.gdn2_strerror(c).decode() for c in range(6)}
    assert len(msgs) == 6
    assert "unknown" in lib.gdn2_strerror(99).decode()


def test_binding_refuses_cpu_tensors():
    import torch
    x = torch.zeros(1, 4, 1, 32)
    with pytest.raises(RuntimeError):
        gdn2.fwd(x, x, x, x, x, x)


def test_output_epilogue_checks_arguments():
    lib = gdn2.load()
    f = P(0x10000)
    s = _shape(B=2, T=100, H=3, dv=128)
    F = ctypes.c_float
    # workspace: one partial dweight row per workgroup (256 threads, 32 lanes a row, 4 rows in flight)
    rows = 2 * 100 * 3
    blocks = min((rows + 31) // 32, 1024)
    assert lib.gdn2_output_bwd_workspace_size(ctypes.byref(s)) == blocks * 128 * 4
    assert lib.gdn2_output_bwd_workspace_size(ctypes.byref(_shape(dv=96))) == ctypes.c_size_t(-1).value
    assert lib.gdn2_output_fwd(ctypes.byref(s), f, f, 0, None, F(-1.0), f, 0, None) == INVALID
    assert lib.gdn2_output_fwd(ctypes.byref(s), f, f, 0, None, F(float("nan")), f, 0, None) == INVALID
    assert lib.gdn2_output_fwd(ctypes.byref(s), f, f, 0, None, F(float("inf")), f, 0, None) == INVALID
    assert lib.gdn2_output_fwd(ctypes.byref(s), f, f, 2, None, F(1e-6), f, 0, None) == UNSUPPORTED
    assert lib.gdn2_output_fwd(ctypes.byref(s), f, f, 0, None, F(1e-6), f, 5, None) == UNSUPPORTED
    assert lib.gdn2_output_fwd(ctypes.byref(s), None, f, 0, None, F(1e-6), f, 0, None) == INVALID
    assert lib.gdn2_output_fwd(ctypes.byref(s), f, f, 0, P(0x10008), F(1e-6), f, 0, None) == INVALID
    assert lib.gdn2_output_fwd(ctypes.byref(_shape(dv=96)), f, f, 0, None, F(1e-6), f, 0, None) == UNSUPPORTED
    need = lib.gdn2_output_bwd_workspace_size(ctypes.byref(s))
    assert lib.gdn2_output_bwd(ctypes.byref(s), f, f, 0, None, F(1e-6), f, f, f, f, None, 0, None) == WORKSPACE
    assert lib.gdn2_output_bwd(ctypes.byref(s), f, f, 0, None, F(1e-6), f, f, f, f, f, need - 1, None) == WORKSPACE
    assert lib.gdn2_output_bwd(ctypes.byref(s), f, f, 0, None, F(1e-6), f, None, f, None, None, 0, None) == INVALID
    assert lib.gdn2_output_bwd(ctypes.byref(s), f, f, 1, None, F(-0.5), f, f, f, None, None, 0, None) == INVALID


@cus_256
def test_sweeps_entry_checks_arguments_and_fusion_rule():
    lib = gdn2.load()
    f = P(0x10000)
    s = _shape()
    # factors, v, w, S0, dO, dS_final, o, S_final, states, dstates, dS0: all but S0, dS_final,
    # S_final and dS0 required, and checked before any launch
    args = [f] * 11
    for i in (0, 1, 2, 4, 6, 8, 9):
        a = list(args)
        a[i] = None
        assert lib.gdn2_chunk_sweeps(ctypes.byref(s), *a, None) == INVALID
    a = list(args)
    a[0] = P(0x10008)
    assert lib.gdn2_chunk_sweeps(ctypes.byref(s), *a, None) == INVALID
    assert lib.gdn2_chunk_sweeps(ctypes.byref(_shape(dv=96)), *args, None) == UNSUPPORTED
    # one launch where both sweeps' 64-column tiles take at most one workgroup per CU (256 CUs)
    def fused(**kw):
        return lib.gdn2_chunk_sweeps_fused(ctypes.byref(_shape(**kw)))
    assert fused(B=4, T=4096, H=16, dk=128, dv=128) == 1
    assert fused(B=1, T=16384, H=16, dk=64, dv=128) == 1
    assert fused(B=8, T=2048, H=16, dk=128, dv=128) == 0
    assert fused(B=4, T=4096, H=16, dk=128, dv=128, dt=0) == 0    # fp32 q/k/v
    assert fused(B=4, T=4096, H=16, dk=32, dv=128) == 0
    assert fused(B=4, T=4096, H=16, dk=128, dv=32) == 0
    assert fused(dk=96) == -1


def test_factored_forward_checks_arguments():
    lib = gdn2.load()
    f = P(0x10000)
    s = _shape()
    # factors, v, w required; o and states cannot both be NULL
    assert lib.gdn2_chunk_fwd_factored(ctypes.byref(s), None, f, f, None, f, None, None, None) == INVALID
    assert lib.gdn2_chunk_fwd_factored(ctypes.byref(s), f, None, f, None, f, None, None, None) == INVALID
    assert lib.gdn2_chunk_fwd_factored(ctypes.byref(s), f, f, None, None, f, None, None, None) == INVALID
    assert lib.gdn2_chunk_fwd_factored(ctypes.byref(s), f, f, f, None, None, f, None, None) == INVALID
    assert lib.gdn2_chunk_fwd_factored(ctypes.byref(s), P(0x10008), f, f, None, f, None, None, None) == INVALID
    assert lib.gdn2_chunk_fwd_factored(ctypes.byref(_shape(dv=96)), f, f, f, None, f, None, None, None) == UNSUPPORTED
    # a per-token write gate needs only word alignment; a per-channel one 16 bytes
    assert lib.gdn2_chunk_fwd_factored(ctypes.byref(s), f, f, P(0x10004), None, f, None, None, None) == INVALID


@cus_256
def test_forward_workspace():
    """The forward writes forward-only chunk records first: it needs a workspace of one record
    per (batch, head, chunk) and their flags.  The segment expectations assume 256 CUs, the
    count the library takes when no device answers."""
    lib = gdn2.load()
    f = P(0x10000)
    record = RECORD
    wide = _shape(B=8, T=2048, H=16, dk=128, dv=128)
    need = lib.gdn2_chunk_fwd_workspace_size(ctypes.byref(wide))
    assert need == 8 * 16 * 32 * record + _flags(8 * 16 * 32)
    F = ctypes.c_size_t
    assert lib.gdn2_chunk_fwd(ctypes.byref(wide), f, f, f, f, f, f, None, f, None, None, F(0), None) == WORKSPACE
    assert lib.gdn2_chunk_fwd(ctypes.byref(wide), f, f, f, f, f, f, None, f, None, f, F(need - 1), None) == WORKSPACE
    # few heads: still the record path; with at most one CU in four busy and a long sequence
    # the sequence is split into segments (here 8 of 32 chunks), whose [N | M] blocks and start
    # states follow the records
    seg = 1 * 16 * 8 * 128 * ((128 + 128) + 128) * 4
    assert lib.gdn2_chunk_fwd_workspace_size(ctypes.byref(_shape(B=1, T=16384, H=16, dk=128, dv=128))) == \
        1 * 16 * 256 * record + _flags(16 * 256) + seg
    # the one-call backward splits its state sweep the same way: the same blocks after the
    # states, their gradients and the factor buffer
    long = _shape(B=1, T=16384, H=16, dk=128, dv=128)
    states = 16 * 256 * 128 * 128 * 4
    factors = 16 * 256 * ((128 * 128 + 64 * 128) * 4 + record) + _flags(16 * 256)
    assert lib.gdn2_chunk_bwd_workspace_size(ctypes.byref(long)) == 2 * states + factors + seg
    # few heads but a short sequence (under 64 chunks): no segments
    assert lib.gdn2_chunk_fwd_workspace_size(ctypes.byref(_shape(B=1, T=4000, H=16, dk=128, dv=128))) == \
        1 * 16 * 63 * record + _flags(16 * 63)
    short = _shape(B=1, T=4000, H=16, dk=128, dv=128)
    assert lib.gdn2_chunk_bwd_workspace_size(ctypes.byref(short)) == \
        2 * 16 * 63 * 128 * 128 * 4 + 16 * 63 * ((128 * 128 + 64 * 128) * 4 + record) + _flags(16 * 63)
    # fp32 q/k/v and dv not a multiple of 64: the same records, swept by the four-wave sweep
    items = 8 * 16 * 32
    assert lib.gdn2_chunk_fwd_workspace_size(ctypes.byref(_shape(B=8, T=2048, H=16, dk=128, dv=128, dt=0))) == \
        items * record + _flags(items)
    assert lib.gdn2_chunk_fwd_workspace_size(ctypes.byref(_shape(B=8, T=2048, H=16, dk=128, dv=32))) == \
        items * record + _flags(items)
    # dk = 32: the smaller record of that width
    rec32 = (6 * 64 * 32 * 2 + 2 * 64 * 64 * 2 + 2 * 16 * 64 * 16 + 4 * 32 * 4 + 32 * 4 + 255) // 256 * 256
    assert lib.gdn2_chunk_fwd_workspace_size(ctypes.byref(_shape(B=8, T=2048, H=16, dk=32, dv=128))) == \
        items * rec32 + _flags(items)



@cus_256
def test_fused_forward_output_workspace_and_checks():
    """gdn2_chunk_fwd_output: with no device answering, a shape whose heads span several
    workgroups cannot be shown resident, so it takes the unfused route (gdn2_chunk_fwd's
    workspace, then o); one value tile per head (dv 64 on 64-column tiles) fuses without a
    cooperative launch: the records, then the row-sum words (a ring of two chunk slots of 2
    words per row and head) and the 256-byte counter slot.  Argument checks come before any
    launch."""
    lib = gdn2.load()
    f = P(0x10000)
    F, Z = ctypes.c_float, ctypes.c_size_t
    unf = _shape(B=8, T=2048, H=16, dk=128, dv=128, dt=0)          # fp32 q/k/v
    fw = lib.gdn2_chunk_fwd_workspace_size(ctypes.byref(unf))
    assert lib.gdn2_chunk_fwd_output_fused(ctypes.byref(unf)) == 0
    assert lib.gdn2_chunk_fwd_output_workspace_size(ctypes.byref(unf)) == \
        (fw + 255) // 256 * 256 + 8 * 2048 * 16 * 128 * 4
    one = _shape(B=3, T=70, H=50, dk=128, dv=64)                    # 150 heads: 64-column tiles, one a head
    items = 3 * 50 * 2
    assert lib.gdn2_chunk_fwd_output_fused(ctypes.byref(one)) == 1
    assert lib.gdn2_chunk_fwd_output_workspace_size(ctypes.byref(one)) == \
        items * RECORD + _flags(items) + 3 * 50 * 2 * 2 * 64 * 8 + 256
    assert lib.gdn2_chunk_fwd_output_workspace_size(ctypes.byref(_shape(dv=96))) == ctypes.c_size_t(-1).value
    s = one
    need = lib.gdn2_chunk_fwd_output_workspace_size(ctypes.byref(s))

    def call(g=f, gdt=0, wt=None, eps=1e-6, y=f, ydt=0, ws=f, nb=need, q=f):
        return lib.gdn2_chunk_fwd_output(ctypes.byref(s), q, f, f, f, f, f, None, g, gdt, wt, F(eps), y, ydt, None,
                                         ws, Z(nb), None)
    assert call(g=None) == INVALID
    assert call(y=None) == INVALID
    assert call(q=None) == INVALID
    assert call(eps=-1.0) == INVALID
    assert call(eps=float("nan")) == INVALID
    assert call(gdt=2) == UNSUPPORTED
    assert call(ydt=3) == UNSUPPORTED
    assert call(wt=P(0x10008)) == INVALID
    assert call(ws=None) == WORKSPACE
    assert call(nb=need - 1) == WORKSPACE
