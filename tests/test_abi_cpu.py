"""The C-ABI boundary without a GPU: the library loads, exports every symbol
its header declares, sizes workspaces consistently, and rejects bad
arguments before any launch (no compute call is made here)."""
import ctypes
import json
import os
import re

import pytest

from mla_paged_latent_03_amd import binding, workloads as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla_decode.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.LIB_PATH):
        from mla_paged_latent_03_amd import build
        build.build()
    return binding.load()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w\s\*]*?\b(mla_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("mla_decode", "mla_decode_fp8", "mla_sparse_decode", "mla_workspace_size", "mla_num_kv_splits",
              "mla_status_string"):
        assert n in names, n


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), "missing export %s" % name
        assert ctypes.cast(getattr(lib, name), ctypes.c_void_p).value


def test_status_strings(lib):
    assert binding.status_string(0) == "ok"
    assert binding.status_string(3) == "workspace too small"
    assert binding.status_string(99) == "unknown status"


def _expected_workspace(B, T, H, s, ws):
    """Partials [B, T*H, s, 513] fp32; a single-launch call adds two 8-byte
    words per (sequence, row block) after them (16-byte aligned)."""
    if s == 1:
        return ws == 0
    partials = B * T * H * s * 513 * 4
    if ws == partials:
        return True
    sync = ws - (partials + 15) // 16 * 16
    row_blocks = -(-T * H // 32)                    # at most one group per 32 rows
    return sync > 0 and sync % 16 == 0 and sync <= 16 * B * row_blocks


@pytest.mark.parametrize("B,T,H,L,K,fp8", [
    (2, 1, 16, 300, 0, False), (128, 1, 16, 8192, 0, False), (64, 4, 32, 80000, 0, True),
    (32, 8, 128, 32768, 0, False), (64, 1, 128, 65536, 2048, False), (3, 2, 24, 5000, 300, False)])
def test_workspace_matches_split_count(lib, B, T, H, L, K, fp8):
    s = binding.num_kv_splits(B, T, H, L, K, fp8)
    assert 1 <= s <= binding.MAX_KV_SPLITS
    ws = binding.workspace_size(B, T, H, L, K, fp8, 0)
    assert _expected_workspace(B, T, H, s, ws), (s, ws)
    for forced in (1, 2, 7):
        ws = binding.workspace_size(B, T, H, L, K, fp8, forced)
        assert _expected_workspace(B, T, H, forced, ws), (forced, ws)


def test_heuristic_fills_the_chip(lib):
    # Dense calls: the split count is costed for sequences of max_seq_len and
    # each sequence then gets twice as many partial slots, so that the device
    # can cut long sequences of a mixed batch into more, equal pieces.
    # The 80k-token MTP-3 fp8 batch: 64 sequences x 1 row block -> 4 pieces each = 256 workgroups.
    assert binding.num_kv_splits(64, 4, 32, 80000, 0, True) == 8
    # 128 one-wave sequences: 4 pieces each = 512 workgroups, two per compute unit.
    assert binding.num_kv_splits(128, 1, 16, 8192, 0, False) == 8
    # Never more slots than pages.
    assert binding.num_kv_splits(2, 1, 16, 300, 0, False) == 5
    # Sparse top-2048 over 64 sequences: 4 splits of 512 indices = 256 four-wave workgroups
    # (narrower row blocks would read every gathered row once per block).
    assert binding.num_kv_splits(64, 1, 128, 65536, 2048, False) == 4
    # A chip already full of units takes one split: partials would only add traffic.
    assert binding.num_kv_splits(256, 4, 32, 700, 0, False) == 1
    assert binding.num_kv_splits(256, 8, 128, 32768, 0, False) == 1
    # A matrix-bound batch (eight row blocks per sequence) that fills one round
    # of workgroups but not two: two pieces per sequence, run longest first.
    assert binding.num_kv_splits(32, 8, 128, 32768, 0, False) == 2
    assert binding.num_kv_splits(63, 8, 128, 32768, 0, False) == 2
    # ... but not once the batch fills two rounds, nor with fewer than four row blocks.
    assert binding.num_kv_splits(64, 8, 128, 32768, 0, False) == 1
    assert binding.num_kv_splits(128, 2, 128, 32768, 0, False) == 1
    # A top-k list longer than one workgroup's index table forces splits.
    assert binding.num_kv_splits(1, 1, 16, 10000, 5000, False) >= 5


def test_launch_waves_follow_the_row_block_rules(lib):
    # 128 rows and enough units to fill the chip: one four-wave row block.
    assert binding.launch_waves(64, 4, 32, 80000, 0, True) == 4
    assert binding.launch_waves(32, 8, 128, 32768, 0, False) == 4
    assert binding.launch_waves(256, 1, 128, 300, 0, False) == 4
    assert binding.launch_waves(64, 1, 128, 65536, 2048, False) == 4
    # 16 rows per sequence: a dense call still takes two waves (the second has
    # no rows but shares each tile's DMA); a sparse one takes one.
    assert binding.launch_waves(128, 1, 16, 8192, 0, False) == 2
    assert binding.launch_waves(128, 1, 16, 8192, 0, True) == 2
    assert binding.launch_waves(128, 1, 16, 65536, 2048, False) == 1
    # Few short sequences: narrower row blocks (and splits) fill more of the chip.
    assert binding.launch_waves(4, 1, 64, 300, 0, False) == 1
    # 64 rows and units enough for two workgroups per compute unit: two waves.
    assert binding.launch_waves(512, 1, 64, 300, 0, False) == 2
    assert binding.launch_waves(1, 0, 16, 100) == 0


def test_invalid_sizes_are_rejected(lib):
    assert binding.num_kv_splits(1, 0, 16, 100) == 0
    assert binding.num_kv_splits(1, 9, 16, 100) == 0
    assert binding.num_kv_splits(1, 1, 0, 100) == 0
    assert binding.workspace_size(1, 1, 16, 100, 0, False, 257) == 0
    assert binding.workspace_size(1, 1, 16, 5000, 4096, False, 1) == 0   # K / splits above the index table


FAKE = 0x10000   # aligned, never dereferenced: every call below fails validation first


def _call_dense(lib, **kw):
    a = dict(q_nope=FAKE, q_pe=FAKE, kv=FAKE, bt=FAKE, sl=FAKE, B=2, T=1, H=16, NB=10, P=64, MB=5, msl=300,
             scale=0.07, out=FAKE, odt=0, lse=FAKE, ws=None, wsb=0, splits=1)
    a.update(kw)
    return lib.mla_decode(a["q_nope"], a["q_pe"], a["kv"], a["bt"], a["sl"], a["B"], a["T"], a["H"], a["NB"],
                          a["P"], a["MB"], a["msl"], a["scale"], a["out"], a["odt"], a["lse"], a["ws"], a["wsb"],
                          a["splits"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(T=0), binding.MLA_ERR_INVALID_ARGUMENT),
    (dict(T=9), binding.MLA_ERR_INVALID_ARGUMENT),
    (dict(H=0), binding.MLA_ERR_INVALID_ARGUMENT),
    (dict(P=32), binding.MLA_ERR_UNSUPPORTED),
    (dict(q_nope=None), binding.MLA_ERR_INVALID_ARGUMENT),
    (dict(out=None), binding.MLA_ERR_INVALID_ARGUMENT),
    (dict(bt=None), binding.MLA_ERR_INVALID_ARGUMENT),
    (dict(q_pe=FAKE + 8), binding.MLA_ERR_INVALID_ARGUMENT),     # misaligned
    (dict(odt=7), binding.MLA_ERR_INVALID_ARGUMENT),
    (dict(splits=300), binding.MLA_ERR_INVALID_ARGUMENT),
    (dict(splits=-1), binding.MLA_ERR_INVALID_ARGUMENT),
    (dict(scale=float("nan")), binding.MLA_ERR_INVALID_ARGUMENT),
    (dict(scale=0.0), binding.MLA_ERR_INVALID_ARGUMENT),       # the row reference needs a positive scale
    (dict(scale=-0.07), binding.MLA_ERR_INVALID_ARGUMENT),
    (dict(MB=0), binding.MLA_ERR_INVALID_ARGUMENT),
    (dict(splits=2, ws=FAKE, wsb=2 * 16 * 2 * 513 * 4 - 1), binding.MLA_ERR_WORKSPACE_TOO_SMALL),
    (dict(splits=2, ws=None, wsb=0), binding.MLA_ERR_WORKSPACE_TOO_SMALL),
])
def test_dense_argument_errors(lib, kw, status):
    assert _call_dense(lib, **kw) == status


def test_empty_batch_is_a_no_op(lib):
    assert _call_dense(lib, B=0, q_nope=None, out=None) == binding.MLA_OK


def test_stage_one_only_needs_explicit_splits(lib):
    assert _call_dense(lib, out=None, lse=None, splits=1) == binding.MLA_ERR_INVALID_ARGUMENT
    assert _call_dense(lib, out=None, lse=None, splits=0) == binding.MLA_ERR_INVALID_ARGUMENT
    assert _call_dense(lib, out=None, lse=FAKE, splits=2, ws=FAKE, wsb=1 << 20) == binding.MLA_ERR_INVALID_ARGUMENT
    assert _call_dense(lib, out=None, lse=None, splits=2, ws=None, wsb=0) == binding.MLA_ERR_WORKSPACE_TOO_SMALL


def test_merge_partials_errors(lib):
    f = lib.mla_merge_partials
    assert f(FAKE, 10, 0, FAKE, 0, None, None) == binding.MLA_ERR_INVALID_ARGUMENT
    assert f(FAKE, 10, 257, FAKE, 0, None, None) == binding.MLA_ERR_INVALID_ARGUMENT
    assert f(FAKE, -1, 2, FAKE, 0, None, None) == binding.MLA_ERR_INVALID_ARGUMENT
    assert f(None, 10, 2, FAKE, 0, None, None) == binding.MLA_ERR_INVALID_ARGUMENT
    assert f(FAKE, 10, 2, FAKE + 4, 0, None, None) == binding.MLA_ERR_INVALID_ARGUMENT
    assert f(FAKE, 10, 2, FAKE, 5, None, None) == binding.MLA_ERR_INVALID_ARGUMENT
    assert f(None, 0, 2, None, 0, None, None) == binding.MLA_OK


def test_fp8_scale_errors(lib):
    for qs, ks in ((0.0, 1.0), (1.0, -1.0), (float("inf"), 1.0)):
        st = lib.mla_decode_fp8(FAKE, FAKE, FAKE, FAKE, FAKE, 2, 1, 16, 10, 64, 5, 300, 0.07, qs, ks, FAKE, 0,
                                FAKE, None, 0, 1, None)
        assert st == binding.MLA_ERR_INVALID_ARGUMENT


def test_sparse_errors(lib):
    args = [FAKE, FAKE, FAKE, FAKE, FAKE]
    tail = [2, 1, 16, 10, 64, 5, 300, 0.07, FAKE, 0, FAKE, None, 0, 1, None]
    assert lib.mla_sparse_decode(*args, None, 64, *tail) == binding.MLA_ERR_INVALID_ARGUMENT   # no indices
    assert lib.mla_sparse_decode(*args, FAKE, 0, *tail) == binding.MLA_ERR_INVALID_ARGUMENT    # K = 0
    big = [2, 1, 16, 10, 64, 5, 300, 0.07, FAKE, 0, FAKE, None, 0, 1, None]
    assert lib.mla_sparse_decode(*args, FAKE, 4096, *big) == binding.MLA_ERR_UNSUPPORTED      # 4096 / 1 split


# ------------------------------------------------------------------ inline-asm hazard scan

_DMA = "buffer_load_dwordx4 v1, s[8:11], s12 offen lds"


def _asm(*lines):
    return "\n".join("\t" + l for l in lines)


def test_asm_hazard_scan_flags_m0_and_sgpr_hazards():
    """The build-time scan of the compiled kernels: an LDS DMA in inline asm
    needs 1 wait state after an SALU write of M0 and 5 after a VALU write of
    an SGPR it reads; the compiler's own memory instructions are not its
    concern."""
    from mla_paged_latent_03_amd import asm_hazards as hz
    clean = _asm("s_mov_b32 m0, s1", ";;#ASMSTART", "s_nop 0", _DMA, ";;#ASMEND")
    assert hz.scan(clean) == []
    no_m0_wait = _asm("s_mov_b32 m0, s1", ";;#ASMSTART", _DMA, ";;#ASMEND")
    assert len(hz.scan(no_m0_wait)) == 1
    fresh_sgpr = _asm("v_readfirstlane_b32 s9, v0", "s_mov_b32 m0, s1", ";;#ASMSTART", "s_nop 0", _DMA, ";;#ASMEND")
    assert len(hz.scan(fresh_sgpr)) == 1
    fresh_soffset = _asm("v_readlane_b32 s12, v254, 3", "s_nop 1", "s_mov_b32 m0, s1", ";;#ASMSTART", "s_nop 0",
                         _DMA, ";;#ASMEND")
    assert len(hz.scan(fresh_soffset)) == 1
    settled = _asm("v_readfirstlane_b32 s9, v0", ";;#ASMSTART", "s_nop 4", ";;#ASMEND", "s_mov_b32 m0, s1",
                   ";;#ASMSTART", "s_nop 0", _DMA, ";;#ASMEND")
    assert hz.scan(settled) == []
    compiler_owned = _asm("v_readfirstlane_b32 s9, v0", "buffer_load_dword v2, v3, s[8:11], 0 offen")
    assert hz.scan(compiler_owned) == []
    sparse = _asm("s_add_i32 m0, s37, 0x400", ";;#ASMSTART", "global_load_lds_dwordx4 v[2:3], off", ";;#ASMEND")
    assert len(hz.scan(sparse)) == 1
    # The forms the kernels issue carry the non-temporal hint; the scan must still see them.
    nt_dense = _asm("s_mov_b32 m0, s1", ";;#ASMSTART", "buffer_load_dwordx4 v1, s[8:11], s12 offen nt lds", ";;#ASMEND")
    assert len(hz.scan(nt_dense)) == 1
    nt_sparse = _asm("s_add_i32 m0, s37, 0x400", ";;#ASMSTART", "global_load_lds_dwordx4 v[2:3], off nt",
                     ";;#ASMEND")
    assert len(hz.scan(nt_sparse)) == 1


def test_asm_hazard_scan_follows_branches_into_a_block():
    """A block entered by a branch: the fall-through path into it has its
    wait states, the branch path does not (the hazard class of the fault
    fixed by the s_nop in the descriptor set-up).  Also a loop back-edge,
    and an unconditional branch that ends the fall-through path."""
    from mla_paged_latent_03_amd import asm_hazards as hz
    branch_entered = _asm("v_readfirstlane_b32 s9, v0", "s_cbranch_scc1 .LBB0_2", "s_nop 4", "s_mov_b32 m0, s1",
                          ".LBB0_2:", ";;#ASMSTART", "s_nop 0", _DMA, ";;#ASMEND")
    found = hz.scan(branch_entered)
    assert len(found) == 1 and "v_readfirstlane_b32 s9" in found[0]
    both_settled = _asm("v_readfirstlane_b32 s9, v0", "s_nop 4", "s_cbranch_scc1 .LBB0_2", "s_nop 4",
                        "s_mov_b32 m0, s1", ".LBB0_2:", ";;#ASMSTART", "s_nop 0", _DMA, ";;#ASMEND")
    assert hz.scan(both_settled) == []
    back_edge = _asm("s_mov_b32 m0, s1", "s_nop 4", ".LBB0_1:", ";;#ASMSTART", "s_nop 0", _DMA, ";;#ASMEND",
                     "s_add_u32 s20, s20, 1", "v_readlane_b32 s12, v5, 0", "s_cbranch_scc1 .LBB0_1")
    found = hz.scan(back_edge)
    assert len(found) == 1 and "v_readlane_b32 s12" in found[0]
    no_fallthrough = _asm("v_readfirstlane_b32 s9, v0", "s_branch .LBB0_3", ".LBB0_2:", ";;#ASMSTART", "s_nop 0",
                          _DMA, ";;#ASMEND", ".LBB0_3:", "s_endpgm")
    assert hz.scan(no_fallthrough) == []


def test_noalloc_refuses_partials_beyond_its_static_buffer(lib):
    """mla_decode_fp8_noalloc sizes the plan before anything else: partials
    over 64 MiB are refused with their own status, before any HIP call (the
    pointers here are never dereferenced)."""
    fake = ctypes.c_void_p(0x1000)
    B, T, H, L = 64, 4, 32, 80000
    assert binding.workspace_size(B, T, H, L, 0, True, 8) > binding.STATIC_SCRATCH_BYTES
    st = lib.mla_decode_fp8_noalloc(fake, fake, fake, fake, fake, B, T, H, 100, 64, 1250, L, 0.07, 1.0, 1.0, fake,
                                    0, fake, 8, None)
    assert st == binding.MLA_ERR_SCRATCH_LIMIT
    assert "static" in binding.status_string(st)
    # invalid arguments keep their usual status
    st = lib.mla_decode_fp8_noalloc(fake, fake, fake, fake, fake, B, 9, H, 100, 64, 1250, L, 0.07, 1.0, 1.0, fake,
                                    0, fake, 2, None)
    assert st == binding.MLA_ERR_INVALID_ARGUMENT


# ------------------------------------------------------------------ dense un-absorbed MHA route

def test_dense_mha_workspace_formula(lib):
    """K_nope [B, H, Lpad, 128] and V^T [B, H, 128, Lpad] bf16, Lpad = max_seq_len
    rounded up to 128."""
    for B, H, L in ((2, 16, 300), (1, 1, 1), (3, 128, 8192), (4, 8, 0), (1, 2, 128), (1, 2, 129)):
        lpad = (L + 127) // 128 * 128
        assert binding.dense_mha_workspace_size(B, H, L) == 2 * B * H * lpad * 128 * 2
    assert binding.dense_mha_workspace_size(-1, 16, 100) == 0
    assert binding.dense_mha_workspace_size(1, 0, 100) == 0
    assert binding.dense_mha_workspace_size(1, 16, -5) == 0


def _call_mha(lib, **kw):
    a = dict(q=FAKE, qpe=FAKE, kv=FAKE, bt=FAKE, sl=FAKE, wk=FAKE, wv=FAKE, B=2, T=4, H=16, NB=10, P=64, MB=5,
             msl=300, scale=0.07, out=FAKE, odt=0, lse=FAKE, ws=FAKE, wsb=1 << 30)
    a.update(kw)
    return lib.mla_dense_mha(a["q"], a["qpe"], a["kv"], a["bt"], a["sl"], a["wk"], a["wv"], a["B"], a["T"], a["H"],
                             a["NB"], a["P"], a["MB"], a["msl"], a["scale"], a["out"], a["odt"], a["lse"], a["ws"],
                             a["wsb"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(T=0), binding.MLA_ERR_INVALID_ARGUMENT),
    (dict(T=binding.MHA_MAX_Q_LEN + 1), binding.MLA_ERR_INVALID_ARGUMENT),
    (dict(H=0), binding.MLA_ERR_INVALID_ARGUMENT),
    (dict(P=32), binding.MLA_ERR_UNSUPPORTED),
    (dict(wk=None), binding.MLA_ERR_INVALID_ARGUMENT),
    (dict(wv=FAKE + 2), binding.MLA_ERR_INVALID_ARGUMENT),
    (dict(q=None), binding.MLA_ERR_INVALID_ARGUMENT),
    (dict(odt=3), binding.MLA_ERR_INVALID_ARGUMENT),
    (dict(MB=0), binding.MLA_ERR_INVALID_ARGUMENT),
    (dict(scale=float("inf")), binding.MLA_ERR_INVALID_ARGUMENT),
    (dict(scale=0.0), binding.MLA_ERR_INVALID_ARGUMENT),
    (dict(scale=-0.07), binding.MLA_ERR_INVALID_ARGUMENT),
    (dict(wsb=2 * 2 * 16 * 384 * 128 * 2 - 1), binding.MLA_ERR_WORKSPACE_TOO_SMALL),
    (dict(B=65535, H=1024, msl=1 << 24, wsb=1 << 62), binding.MLA_ERR_UNSUPPORTED),
    (dict(ws=None), binding.MLA_ERR_INVALID_ARGUMENT),
    (dict(ws=FAKE + 8), binding.MLA_ERR_INVALID_ARGUMENT),
])
def test_dense_mha_argument_errors(lib, kw, status):
    assert _call_mha(lib, **kw) == status


def test_dense_mha_empty_batch_is_a_no_op(lib):
    assert _call_mha(lib, B=0, q=None, out=None, ws=None, wsb=0) == binding.MLA_OK


def test_product_path_fails_loudly_without_the_library_or_a_gpu(monkeypatch):
    """No CPU fallback: a missing library raises at load, and host tensors are
    refused before anything reaches the C ABI."""
    monkeypatch.setattr(binding, "_lib", None)
    with pytest.raises(ImportError):
        binding.load("/nonexistent/libmla_decode.so")
    monkeypatch.undo()
    inp = wl.make_inputs(1, 16, 1, [40], kv_dtype="bf16", out_dtype="f32", seed=3)
    with pytest.raises(ValueError, match="GPU"):
        binding.decode(inp)


def test_benchmark_reference_library_rejects_bad_arguments():
    """The benchmark's reference library (streaming read, LDS read rate)
    loads and refuses bad arguments before touching a device."""
    path = os.path.join(ROOT, "mla_paged_latent_03_amd", "libmla_stream_ref.so")
    if not os.path.exists(path):
        from mla_paged_latent_03_amd import build
        build.build()
    ref = ctypes.CDLL(path)
    sr = ref.mla_stream_read_reference
    sr.restype = ctypes.c_int
    sr.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    fake = ctypes.c_void_p(1 << 20)                 # never dereferenced: every case fails validation
    assert sr(None, 36864, 1, fake, None) == 1       # no source
    assert sr(fake, 36864, 0, fake, None) == 1       # no workgroups
    assert sr(fake, 1000, 1, fake, None) == 1        # not a whole number of tiles
    assert sr(ctypes.c_void_p((1 << 20) + 8), 36864, 1, fake, None) == 1   # misaligned source
    lr = ref.mla_lds_read_rate_reference
    lr.restype = ctypes.c_int
    lr.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                   ctypes.POINTER(ctypes.c_int), ctypes.c_void_p]
    khz = ctypes.c_int(0)
    assert lr(3, 8, 1, 1, fake, fake, ctypes.byref(khz), None) == 1      # waves not 1, 2, 4, 8 or 16
    assert lr(4, 5, 1, 1, fake, fake, ctypes.byref(khz), None) == 1      # reads in flight not 2, 4, 8 or 16
    assert lr(4, 8, 0, 1, fake, fake, ctypes.byref(khz), None) == 1      # no workgroups
    assert lr(4, 8, 1, 0, fake, fake, ctypes.byref(khz), None) == 1      # no iterations
    assert lr(4, 8, 1, 1, None, fake, ctypes.byref(khz), None) == 1      # no sink
    assert lr(4, 8, 1, 1, fake, fake, None, None) == 1                   # no clock-rate output
