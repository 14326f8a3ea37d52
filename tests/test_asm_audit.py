"""Audit of the gfx950 assembly the library is built from (CPU; hipcc only).

The batch1-cdna README's measurement rules check the generated assembly of
every experiment, because several failure modes (a reduction hoisted out of a
loop, DPP not emitted, a dot instruction lowered to plain arithmetic) give
plausible timings and wrong conclusions.  These checks pin the instructions
each kernel's design relies on, and forbid what must never appear:
  * writes through the scalar data cache (scalar stores, scalar atomics,
    scalar cache write-back or discard);
  * packed fp32 arithmetic (the build disables it);
  * register spills to scratch memory.
"""
import concurrent.futures as cf
import os
import re

import pytest

from memory_bound_decode_gemv_amd import _build


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    d = tmp_path_factory.mktemp("asm")
    srcs = _build.sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        outs = list(ex.map(lambda s: _build.device_asm(s, str(d / (os.path.basename(s) + ".s"))), srcs))
    return {os.path.basename(s): open(o).read() for s, o in zip(srcs, outs)}


def _kernels(text):
    """(mangled name, body) of every kernel in an assembly file."""
    out = []
    for m in re.finditer(r"^(_Z\w+):", text, re.M):
        end = text.find("s_endpgm", m.end())
        out.append((m.group(1), text[m.end():end]))
    return out


def test_every_source_has_kernels(asm):
    for name, text in asm.items():
        if name != "api.hip":
            assert _kernels(text), name


def test_no_scalar_cache_writes(asm):
    bad = re.compile(r"^\s*(s_store|s_buffer_store|s_atomic|s_buffer_atomic|s_dcache_wb|s_dcache_discard|"
                     r"s_scratch_store)", re.M)
    for name, text in asm.items():
        assert not bad.search(text), name


def test_no_packed_fp32(asm):
    bad = re.compile(r"^\s*v_pk_(add|mul|fma|mov)_f32", re.M)
    for name, text in asm.items():
        assert not bad.search(text), name


def test_no_spills_or_scratch(asm):
    for name, text in asm.items():
        for m in re.finditer(r"\.private_segment_fixed_size:\s*(\d+)", text):
            assert int(m.group(1)) == 0, name
        for m in re.finditer(r"\.vgpr_spill_count:\s*(\d+)", text):
            assert int(m.group(1)) == 0, name


def test_dense_gemv_uses_dot2_nontemporal_loads_and_dpp(asm):
    t = asm["gemv_dense.hip"]
    assert "v_dot2_f32_f16" in t or "v_dot2c_f32_f16" in t
    assert "v_dot2_f32_bf16" in t or "v_dot2c_f32_bf16" in t
    assert re.search(r"global_load_dwordx4 .* nt", t)
    assert "row_shr:1" in t and "row_bcast:15" in t and "row_bcast:31" in t


def test_q4_kernels_use_dot4_lds_dma_and_matrix_cores(asm):
    m1 = asm["gemv_q4_0_m1.hip"]
    assert "global_load_lds_dwordx4" in m1
    assert "v_dot4_i32_i8" in m1 or "v_dot4c_i32_i8" in m1
    assert "flat_load" not in m1           # LDS addresses stay LDS addresses
    mf = asm["gemv_q4_0_mfma.hip"]
    assert "v_mfma_i32_16x16x32_i8" in mf
    assert "global_load_lds_dwordx4" in mf
    assert "flat_load" not in mf
    assert not re.search(r"v_accvgpr_read", mf)   # results stay in VGPRs
    un = asm["gemv_m1_units.hip"]
    assert "global_load_lds_dwordx4" in un and "s_barrier" in un
    assert "v_dot4_i32_i8" in un or "v_dot4c_i32_i8" in un
    assert "flat_load" not in un


def test_matrix_core_scale_products_and_private_parts(asm):
    """Both int8 matrix-core kernels take the d8 x d4 scale products from the
    f16 matrix cores; the streaming kernel with one row tile per workgroup
    (template RT = 1) meets its waves only at the row-group start and the
    two-step K-part reduction (3 barriers), the shared-column forms also
    inside the loop."""
    for src in ("gemv_q4_0_mfma.hip", "gemv_qmfma_res.hip"):
        ks = [(n, b) for n, b in _kernels(asm[src]) if "k_qmfma" in n or "k_qres" in n]
        assert ks, src
        for n, b in ks:
            assert "v_mfma_f32_16x16x16_f16" in b, n
    seen = 0
    for n, b in _kernels(asm["gemv_q4_0_mfma.hip"]):
        m = re.search(r"k_qmfma.*?ELi8ELi(\d+)ELi(\d+)ELi(\d+)ELi(\d+)E", n)
        if not m:
            continue
        rt, ks = int(m.group(2)), int(m.group(3))
        if rt == 1:
            assert b.count("s_barrier") == 3, n
            seen += 1
        elif ks > 1:
            assert b.count("s_barrier") > 3, n
    assert seen >= 8


def test_resident_matrix_core_kernel(asm):
    """Weights reach the matrix cores through registers and a per-wave LDS
    transpose (16-byte non-temporal loads, ds_write_b128), the activation
    operands come from LDS, and MFMA results stay in VGPRs."""
    t = asm["gemv_qmfma_res.hip"]
    assert "v_mfma_i32_16x16x32_i8" in t
    assert re.search(r"global_load_dwordx4 .* nt", t)
    assert "ds_write_b128" in t and "ds_read_b128" in t
    assert "global_load_lds" not in t and "flat_load" not in t
    assert not re.search(r"v_accvgpr_read", t)


def test_nf4_row_loop_keeps_loads_in_flight(asm):
    """The NF4 kernels stream rows into registers with the compiler's own
    vmcnt waits; a store or an early exit inside the row loop once made it
    drain every load at the loop head.  No vmcnt(0) may appear in them."""
    seen = 0
    for name, body in _kernels(asm["gemv_nf4.hip"]):
        if "k_nf4I" in name or "k_nf4_rowsI" in name:
            assert "s_waitcnt vmcnt(0)" not in body, name
            seen += 1
    assert seen >= 2


def test_nf4_default_kernel_form(asm):
    """The default NF4 kernel: a code byte's entry comes from one byte permute
    and one 8-byte LDS read, the products are fp32 FMAs (no binary16 dot),
    and four rows are reduced with the permlane swaps."""
    ks = [(n, b) for n, b in _kernels(asm["gemv_nf4.hip"]) if "k_nf4_rowsI" in n]
    assert ks
    for n, b in ks:
        assert "v_perm_b32" in b and "ds_read_b64" in b, n
        assert "v_fmac_f32" in b and "v_dot2" not in b, n
        assert "v_permlane32_swap" in b and "v_permlane16_swap" in b, n


def test_stream_probe_has_no_atomics(asm):
    t = asm["stream_read.hip"]
    assert "global_atomic" not in t
    assert re.search(r"global_load_dwordx4 .* nt", t)


def test_argmax_wave_reduction_on_dpp(asm):
    """The argmax reductions combine the lanes' 64-bit keys with DPP row_shr /
    row_bcast moves, not with LDS-routed shuffles (ds_bpermute / ds_swizzle
    would be the shuffle lowering)."""
    t = asm["argmax.hip"]
    assert "row_shr:1" in t and "row_shr:8" in t and "row_bcast:15" in t and "row_bcast:31" in t
    assert "ds_bpermute" not in t


def test_tiled_kernel_form(asm):
    """The tiled Q4_0 / Q8_0 kernel: weights straight into registers with
    16-byte non-temporal loads (no LDS copy of weights), the activation
    columns by LDS DMA, one int8 MFMA per block (no offset product) or per two
    blocks (the 64-deep form of the pair tiles), the scale products on the
    f16 matrix cores, MFMA results in VGPRs.  The split-K ticket exchange
    uses vector atomics and device-coherent loads and stores, never the
    whole-cache write-back and invalidate of agent-scope fences."""
    t = asm["gemv_tiles.hip"]
    ks = [(n, b) for n, b in _kernels(t) if "k_tilesI" in n]
    assert len(ks) >= 40
    formats = set()
    for n, b in ks:
        m = re.search(r"k_tilesINS0_\d+Tiles(Q4_0|Q8_0)ELi(\d+)E", n)
        assert m, n
        formats.add(m.group(1))
        mp = int(m.group(2))
        assert re.search(r"global_load_dwordx4 .* nt", b), n
        assert "global_load_lds_dwordx4" in b, n
        assert "v_mfma_f32_16x16x16_f16" in b, n
        assert "buffer_wbl2" not in b and "buffer_inv" not in b, n
        assert "global_atomic_add" in b, n
        assert not re.search(r"v_accvgpr_read", b), n
        assert ("v_mfma_i32_16x16x64_i8" in b) == (mp in (8, 24)), n
        assert ("v_mfma_i32_16x16x32_i8" in b) == (mp >= 16), n
    assert formats == {"Q4_0", "Q8_0"}
    # the rearrangement kernels write whole 16-byte slots
    for pack in ("k_q4_tiles_pack", "k_q8_tiles_pack"):
        pk = [b for n, b in _kernels(t) if pack in n]
        assert pk and "global_store_dwordx4" in pk[0], pack
