"""The hand-ordered parts of the kernels (asm MFMAs, asm loads into LDS and
registers) rely on wait states and wait counts the compiler cannot see.  These
tests build the device assembly with the package's own flags and scan it
(`tests/isa_scan.py`).  CPU only: hipcc cross-compiles for gfx950."""
import concurrent.futures as cf
import os
import re
import shutil
import subprocess

import pytest

from attention_flash_sdpa_amd import build as B

import isa_scan  # tests/ is on sys.path (pytest prepends the test file's folder)

pytestmark = pytest.mark.skipif(not os.path.exists(B.HIPCC) and shutil.which("hipcc") is None,
                                reason="hipcc not available")

SOURCES = ["prefill.hip", "prefill_cached.hip", "prefill_split.hip", "prefill_o2.hip", "prefill_fp8.hip",
           "decode.hip"]


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    d = tmp_path_factory.mktemp("isa")

    def compile_one(src):
        out = d / (src + ".s")
        cmd = [B.HIPCC, "-x", "hip", *B.COMMON, *B.DEVICE, *B.EXTRA.get(src, []), "--cuda-device-only", "-S",
               os.path.join(B.CSRC, src), "-o", str(out)]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        return src, out.read_text()

    with cf.ThreadPoolExecutor(max_workers=6) as ex:
        return dict(ex.map(compile_one, SOURCES))


def _functions(text, marker):
    """The assembly of the kernels whose symbol contains `marker`."""
    parts = []
    for m in re.finditer(r"^(_ZN4sdpa\w+):", text, re.M):
        if marker in m.group(1):
            parts.append(text[m.start():text.index(".Lfunc_end", m.end())])
    return "\n".join(parts)


@pytest.mark.parametrize("src", ["prefill.hip", "prefill_cached.hip", "prefill_split.hip"])
def test_hand_ordered_mfma_results_drained(asm, src):
    # only the one-wave kernel orders its MFMAs by hand (inline assembly);
    # the compiler places the wait states of builtin MFMAs itself
    bad, n = isa_scan.mfma_result_waits(_functions(asm[src], "14prefill_kernel"))
    assert n > 1000 and not bad, bad[:5]


@pytest.mark.parametrize("src", SOURCES)
def test_vector_writes_before_mfma_inputs(asm, src):
    bad, n = isa_scan.valu_to_mfma_inputs(asm[src])
    assert n > 0 and not bad, bad[:5]


@pytest.mark.parametrize("src", SOURCES)
def test_asm_lds_reads_waited_for(asm, src):
    # an LDS read written in inline asm is invisible to the compiler's wait
    # count pass: nothing (a register copy or spill included) may touch its
    # result before a wait that covers it, on any path
    bad, n = isa_scan.asm_lds_reads_waited(asm[src])
    assert n > 0 and not bad, bad[:5]


@pytest.mark.parametrize("src", SOURCES)
def test_global_load_results_waited_for(asm, src):
    # loads the compiler does not count (Q fragments, the additive bias) are
    # waited for explicitly: no copy or spill of their registers may come first
    bad, n = isa_scan.global_loads_waited(asm[src])
    assert not bad, bad[:5]


@pytest.mark.parametrize("src", SOURCES)
def test_transcendental_results_waited_for(asm, src):
    bad, n = isa_scan.trans_result_use(asm[src])
    assert n > 0 and not bad, bad[:5]


@pytest.mark.parametrize("src", ["prefill.hip", "prefill_split.hip", "prefill_o2.hip"])
def test_lds_dma_scalar_base_wait_states(asm, src):
    bad, n = isa_scan.lds_dma_scalar_base(asm[src])
    assert n > 0 and not bad, bad[:5]


@pytest.mark.parametrize("src", ["prefill_cached.hip", "prefill_fp8.hip", "decode.hip"])
def test_lds_dma_m0_wait_state(asm, src):
    bad, _ = isa_scan.lds_dma_scalar_base(asm[src])
    assert not bad, bad[:5]


@pytest.mark.parametrize("src", ["prefill.hip", "prefill_split.hip", "prefill_o2.hip"])
def test_untracked_q_loads_waited_for(asm, src):
    bad, n = isa_scan.untracked_loads_waited(asm[src])
    assert n > 0 and not bad, bad[:5]


def test_untracked_load_scan_on_hand_written_code():
    """The scan itself: a register of a load in flight read before the wait is
    caught, as is a later load addressed by one; its earlier value read
    before the load issues, and any read after the wait, are not."""
    def fn(*ins):
        return "_ZN4sdpa1fEv:\n" + "\n".join("\t" + i for i in ins) + "\n.Lfunc_end0:\n"

    ok = fn("v_mov_b32_e32 v5, v1",
            "global_load_dwordx4 v[0:3], v[8:9], off",
            "v_accvgpr_write_b32 a1, v4",          # not a load destination
            "global_load_dwordx4 v[4:7], v[8:9], off offset:16",
            "s_waitcnt vmcnt(0)",
            "v_add_f32_e32 v10, v0, v4")
    assert isa_scan.untracked_loads_waited(ok) == ([], 2)
    read = fn("global_load_dwordx4 v[0:3], v[8:9], off", "v_accvgpr_write_b32 a1, v2", "s_waitcnt vmcnt(0)")
    assert len(isa_scan.untracked_loads_waited(read)[0]) == 1
    addr = fn("global_load_dwordx4 v[0:3], v[8:9], off", "global_load_dwordx4 v[4:7], v[2:3], off",
              "s_waitcnt vmcnt(0)")
    assert len(isa_scan.untracked_loads_waited(addr)[0]) == 1
