"""The gfx950 assembly of the finalize kernels, checked on the CPU.

csrc/finalize_kernels.hip is compiled to device assembly with the library's
own flags, and the claims the design rests on are checked instruction by
instruction:

- no matrix-core (MFMA) instructions: the path is a gather-reduce, not a
  contraction; no packed FP32 instructions (the build turns them off); no
  scratch memory and no register spills in any of the kernels;
- no scalar-cache memory writes of any kind;
- the prefill kernel (index map, FP32 weights, RMSNorm, top-k 8, one vector
  per thread) reads its slot metadata with scalar loads, issues all 8 row
  gathers as non-temporal 16-byte loads, reduces across lanes with DPP,
  converts with the packed BF16 convert and stores through a buffer
  resource with the sc1 policy;
- an index-map token with more slots than fit streams them through the
  rolling window: every slot's rows are one unconditional buffer load per
  vector, and the wait before each slot's FMAs leaves the rest of the window
  in flight;
- a token-major token with more slots than fit arrives in batches: the
  second batch's loads follow a full drain of the first's;
- a team with more threads than vectors (hidden / 256 odd: the last half
  wave idle) reads its rows through buffer loads bounded at the row's end,
  and issues every gather of the batch before its first wait;
- a wave holding several tokens (hidden 256: four tokens at top-k 1, two
  at top-k 2-7; hidden 512 at top-k 1: two) issues every slot's row loads, one 16-byte load per
  vector per lane, before its first wait, keeps no per-token array in LDS,
  and has no spills.
"""
import os
import re
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "moe_expert_output_finalize_amd")
CSRC = os.path.join(PKG, "csrc")


def _build_module():
    import importlib.util
    spec = importlib.util.spec_from_file_location("_mf_build", os.path.join(PKG, "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.fixture(scope="module")
def asm():
    b = _build_module()
    if not os.path.exists(b.hipcc()):
        pytest.skip("needs hipcc")
    flags = [f for f in b.HIPCC_FLAGS if f not in ("-shared", "-fPIC")]
    with tempfile.TemporaryDirectory() as d:
        out = os.path.join(d, "finalize_kernels.s")
        cmd = [b.hipcc(), *flags, "--cuda-device-only", "-S", "-I", os.path.join(ROOT, "include"),
               "-I", CSRC, os.path.join(CSRC, "finalize_kernels.hip"), "-o", out]
        p = subprocess.run(cmd, capture_output=True, text=True, timeout=900)
        assert p.returncode == 0, p.stderr[-3000:]
        with open(out) as f:
            return f.read()


def kernel_name(layout, w_bf16, epi, kc, vpt, exact, tpw=1):
    """Mangled name of
    finalize_kernel<Layout(layout), w_bf16, Epilogue(epi), kc, vpt, exact, tpw>."""
    num = (lambda v: f"n{-v}" if v < 0 else str(v))
    b = (lambda v: "1" if v else "0")
    return (f"_ZN2mf12_GLOBAL__N_115finalize_kernelILNS_6LayoutE{layout}ELb{b(w_bf16)}"
            f"ELNS_8EpilogueE{epi}ELi{num(kc)}ELi{vpt}ELb{b(exact)}ELi{tpw}"
            f"EEEvNS_12FinalizeArgsE")


def body(asm_text, name):
    start = asm_text.index(f"\n{name}:")
    end = asm_text.index("s_endpgm", start)
    return asm_text[start:end]


def metadata(asm_text):
    """Kernel name -> {key: int} from the code-object metadata notes."""
    out = {}
    for block in re.split(r"\n\s+- \.", asm_text.split("amdhsa.kernels:", 1)[1]):
        m = re.search(r"\.name:\s+(\S+)", block)
        if not m or "finalize_kernel" not in m.group(1):
            continue
        out[m.group(1)] = {k: int(v) for k, v in
                           re.findall(r"\.(\w+):\s+(\d+)\s*$", block, flags=re.M)}
    return out


def test_no_matrix_cores_packed_fp32_or_scratch(asm):
    assert "v_mfma" not in asm
    assert not re.search(r"v_pk_(add|mul|fma)_f32", asm)
    meta = metadata(asm)
    assert len(meta) >= 200, len(meta)
    for name, m in meta.items():
        assert m.get("private_segment_fixed_size", 0) == 0, name
        assert m.get("vgpr_spill_count", 0) == 0 and m.get("sgpr_spill_count", 0) == 0, name


def test_no_scalar_cache_writes(asm):
    assert not re.search(r"^\s*s_(buffer_)?(store|atomic)", asm, flags=re.M)
    assert not re.search(r"^\s*s_dcache_wb", asm, flags=re.M)


def test_prefill_kernel_instruction_mix(asm):
    k = body(asm, kernel_name(0, False, 1, 8, 1, True))
    meta = metadata(asm)[kernel_name(0, False, 1, 8, 1, True)]
    rows = re.findall(r"global_load_dwordx4 .* nt$", k, flags=re.M)
    assert len(rows) == 8, rows                       # one 16-byte vector per slot
    first_row = re.search(r"global_load_dwordx4 .* nt$", k, flags=re.M).start()
    assert "s_load_dwordx8" in k[:first_row]          # indices and weights: scalar loads first
    assert all(op in k for op in ("row_half_mirror", "row_mirror", "quad_perm"))
    assert "v_cvt_pk_bf16_f32" in k
    assert re.search(r"buffer_store_dwordx4 .* sc1$", k, flags=re.M)
    assert meta["vgpr_count"] <= 64                   # two 512-thread workgroups fit a CU


def test_rolling_window_keeps_slots_in_flight(asm):
    # index map, FP32 weights, RMSNorm, run-time top-k up to 32, two vectors per thread
    k = body(asm, kernel_name(0, False, 1, -32, 2, True))
    loads = re.findall(r"buffer_load_dwordx4 .* offen nt$", k, flags=re.M)
    assert len(loads) == 64, len(loads)               # 32 slots x 2 vectors, all unconditional
    waits = [int(x) for x in re.findall(r"s_waitcnt vmcnt\((\d+)\)", k)]
    assert max(waits) >= 14                           # 7 more slots' vectors stay in flight


def test_token_major_batches_drain(asm):
    # token major, post-norm, top-k 16, two vectors per thread: two batches of 8 slots
    k = body(asm, kernel_name(1, False, 4, 16, 2, True))
    rows = [m.start() for m in re.finditer(r"global_load_dwordx4 .* nt$", k, flags=re.M)]
    assert len(rows) == 32, len(rows)
    drains = [m.start() for m in re.finditer(r"s_waitcnt vmcnt\(0\)", k)]
    # the first batch's 16 row loads, a full drain, then the second batch's 16
    between = [d for d in drains if rows[15] < d < rows[16]]
    assert between, "no drain between the two batches"


@pytest.mark.parametrize("layout,epi,kc", [(0, 1, -12), (0, 1, -4), (0, 0, 8), (1, 4, -4)])
def test_half_idle_wave_issues_every_gather_first(asm, layout, epi, kc):
    # vectors per thread 1, not exact (hidden 768, 1280, ..., 7936)
    k = body(asm, kernel_name(layout, False, epi, kc, 1, False))
    loads = [m.start() for m in re.finditer(r"buffer_load_dwordx4 .* offen nt$", k, flags=re.M)]
    assert len(loads) == abs(kc), len(loads)
    first_wait = re.search(r"s_waitcnt vmcnt\(\d+\)", k)
    assert first_wait is None or first_wait.start() > loads[-1]


# (layout, epilogue, slot count, vectors per lane, tokens per wave): hidden
# 256 holds 4 tokens of 2 vectors per lane or 2 of 1; hidden 512 2 of 2.
@pytest.mark.parametrize("layout,epi,kc,vpt,tpw", [
    (0, 1, 1, 2, 4), (0, 0, -2, 1, 2), (0, 1, -4, 1, 2), (0, 1, -8, 1, 2), (1, 4, -8, 1, 2),
    (1, 4, 1, 2, 4), (1, 5, -2, 1, 2), (2, 1, 1, 2, 4), (2, 5, 1, 2, 4),
    (0, 1, 1, 2, 2), (0, 0, 1, 2, 2), (1, 4, 1, 2, 2), (2, 1, 1, 2, 2), (2, 5, 1, 2, 2)])
def test_multi_token_wave_issues_every_gather_first(asm, layout, epi, kc, vpt, tpw):
    name = kernel_name(layout, False, epi, kc, vpt, True, tpw)
    k = body(asm, name)
    loads = [m.start() for m in re.finditer(r"global_load_dwordx4 .* nt$", k, flags=re.M)]
    # each lane: vpt vectors of its token's row per slot
    assert len(loads) == abs(kc) * vpt, len(loads)
    first_wait = re.search(r"s_waitcnt vmcnt\(\d+\)", k)
    assert first_wait is None or first_wait.start() > loads[-1]
    # the per-token slot metadata stays in registers (an array the compiler
    # placed in LDS would show as static LDS beyond the norm's 128 bytes)
    assert metadata(asm)[name].get("group_segment_fixed_size", 0) <= 128
