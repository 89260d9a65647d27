"""The compiled kernels' LDS-read waits (CPU: hipcc emits gfx950 assembly).

The NN kernels issue the transposing LDS read as inline assembly that the
compiler's wait-count pass does not track; these tests prove on the compiled
code that no instruction uses such a read's destination before a wait that
covers it, and that no production main loop drains the direct-to-LDS load
pipeline (vmcnt(0)).  The wait analysis itself is pinned on hand-written assembly
with planted mistakes.
"""
import pytest

import isa_waits
from dense_half_precision_amd import build as hbuild


@pytest.fixture(scope="module")
def api_asm(tmp_path_factory):
    out = tmp_path_factory.mktemp("asm") / "hgemm_api.s"
    return open(hbuild.asm("hgemm_api.hip", str(out))).read()


@pytest.fixture(scope="module")
def kernels(api_asm):
    ks = isa_waits.kernel_bodies(api_asm, "_ZN5hgemm")
    assert ks
    return ks


@pytest.fixture(scope="module")
def probe_kernels(tmp_path_factory):
    out = tmp_path_factory.mktemp("asm") / "probe.s"
    asm = open(hbuild.asm("probe.hip", str(out))).read()
    ks = isa_waits.kernel_bodies(asm, "_Z")
    assert ks
    return ks


def test_probe_kernels_no_early_use(probe_kernels):
    """The probes that run the transposing read (inline assembly) too."""
    tr = 0
    for name, lines in probe_kernels.items():
        tr += sum("ds_read_b64_tr_b16" in l for l in lines)
        bad = isa_waits.check_kernel(lines)
        assert not bad, f"{name}: {bad[:5]}"
    assert tr > 0


def test_no_early_use_of_lds_reads(kernels):
    tr = 0
    for name, lines in kernels.items():
        tr += sum("ds_read_b64_tr_b16" in l for l in lines)
        bad = isa_waits.check_kernel(lines)
        assert not bad, f"{name}: {bad[:5]}"
    assert tr > 0  # the NN kernels were checked with their transposing reads


def test_production_loops_keep_loads_in_flight(kernels):
    prod = {n: l for n, l in kernels.items() if n.startswith("_ZN5hgemm11gemm_kernel")}
    assert len(prod) >= 12
    for name, lines in prod.items():
        assert any("Loop Header" in l for l in lines), name
        assert isa_waits.loop_vmcnt_zero(lines) == 0, name


# ---------------------------------------------------------- the wait analysis
def _k(body):
    return ["k:"] + [("\t" + l if not l.startswith(".") else l) for l in body] + ["\ts_endpgm"]


def test_checker_flags_use_before_wait():
    body = ["ds_read_b64_tr_b16 v[0:1], v10 offset:512",
            "v_mfma_f32_16x16x32_f16 a[0:3], v[0:3], v[4:7], a[0:3]"]
    assert isa_waits.check_kernel(_k(body))
    body.insert(1, "s_waitcnt lgkmcnt(0)")
    assert not isa_waits.check_kernel(_k(body))


def test_checker_in_order_retirement():
    body = ["ds_read_b64_tr_b16 v[0:1], v10",
            "ds_read_b128 v[4:7], v11",
            "s_waitcnt lgkmcnt(1)",           # the older (transposing) read is done
            "v_add_u32_e32 v20, v0, v1"]
    assert not isa_waits.check_kernel(_k(body))
    body.append("v_add_u32_e32 v21, v4, v5")  # the younger one may still be in flight
    assert isa_waits.check_kernel(_k(body))


def test_checker_overwrite_and_address_reuse():
    # a VALU write to a register an LDS read will still fill
    assert isa_waits.check_kernel(_k(["ds_read_b128 v[0:3], v8", "v_mov_b32_e32 v2, 0"]))
    # a later LDS read may use a pending destination only as its own destination
    assert not isa_waits.check_kernel(_k(["ds_read_b64 v[0:1], v8", "ds_read_b64 v[0:1], v9",
                                          "s_waitcnt lgkmcnt(0)", "v_mov_b32_e32 v2, v0"]))
    assert isa_waits.check_kernel(_k(["ds_read_b64 v[0:1], v8", "ds_read_b64 v[2:3], v1"]))


def test_checker_follows_the_back_edge():
    """A read issued at the end of a loop body and used at its top is caught
    on the second trip; the exit path is checked too."""
    body = ["s_waitcnt lgkmcnt(0)",
            ".LBB0_1:                                ; =>This Inner Loop Header: Depth=1",
            "v_mfma_f32_16x16x32_f16 a[0:3], v[0:3], v[4:7], a[0:3]",
            "ds_read_b128 v[0:3], v8",
            "s_cbranch_scc0 .LBB0_1",
            "v_mov_b32_e32 v9, 1"]
    assert isa_waits.check_kernel(_k(body))
    fixed = body[:4] + ["s_waitcnt lgkmcnt(0)"] + body[4:]
    assert not isa_waits.check_kernel(_k(fixed))
    assert isa_waits.loop_vmcnt_zero(_k(body)) == 0
    assert isa_waits.loop_vmcnt_zero(_k(body[:3] + ["s_waitcnt vmcnt(0)"] + body[3:])) == 1


def test_partial_sum_stores_read_accumulators_in_place(kernels):
    """The K-segment kernels store their FP32 partial sums with inline assembly
    straight from the accumulator registers.  The compiler does not see those
    stores, so it pads no wait states around them: if it moved accumulators
    through a scratch register range for them (it does when the accumulators
    stay live afterwards), a later write could overwrite store data not yet
    read.  Every such store must read registers of its own."""
    checked = 0
    for name, lines in kernels.items():
        src = isa_waits.acc_store_sources(lines)
        if not src:
            continue
        checked += 1
        dup = {r for r in src if src.count(r) > 1}
        assert not dup, f"{name}: accumulator registers stored more than once: {sorted(dup)[:4]}"
    assert checked >= 20


def test_production_kernels_do_not_spill(api_asm):
    """Every instantiation of the production kernel template with the
    LDS-staged epilogue (all four layouts, tiles, ring depths and launch
    modes) keeps its values in registers: no scratch.  (The register file is full in the
    256 x 256 kernels, 256 accumulators and 256 other registers a lane, so a
    change that raises the pressure anywhere, the epilogue included, shows
    here as spills the main loop may pay for.)"""
    import re
    pat = re.compile(r"\.amdhsa_kernel (_ZN5hgemm11gemm_kernelINS_7TileCfgI((?:Li\d+E){8})EE"
                     r"Li(\d+)ELi(\d+)ELi(\d+)E\S*)")
    checked = 0
    for m in pat.finditer(api_asm):
        cfg = [int(x) for x in re.findall(r"Li(\d+)E", m.group(2))]
        if cfg[3] != 1:  # EPI 1
            continue
        block = api_asm[m.start():m.start() + 4000]
        scratch = int(re.search(r"\.amdhsa_private_segment_fixed_size (\d+)", block).group(1))
        assert scratch == 0, f"{m.group(1)}: {scratch} bytes of scratch"
        checked += 1
    assert checked >= 100

