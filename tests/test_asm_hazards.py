"""The compiled bf16 prefill kernel keeps the hazard rules of its inline-asm MFMAs
(tests/asm_hazards.py): a compiler that reuses an operand register or copies an
unfinished accumulator would corrupt S silently, and nothing else would notice
before a GPU run."""
import os
import shutil
import subprocess

import pytest

import asm_hazards

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _hipcc():
    for c in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    return None


@pytest.fixture(scope="module")
def prefill_asm(tmp_path_factory):
    hipcc = _hipcc()
    if hipcc is None:
        pytest.skip("hipcc not available")
    from token_level_sparse_full_amd import build
    out = str(tmp_path_factory.mktemp("asm") / "attn_prefill_bf16.s")
    src = os.path.join(ROOT, "token_level_sparse_full_amd", "csrc", "attn_prefill_bf16.hip")
    r = subprocess.run([hipcc, *build.FLAGS, "--cuda-device-only", "-S", "-o", out, src],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    with open(out) as f:
        return asm_hazards.functions(f.read())


def test_every_head_count_is_compiled(prefill_asm):
    names = [n for n in prefill_asm if "prefill_bf16_kernel" in n]
    assert len(names) == 20, names   # H in {1, 2, 4, 8, 16} x two passes x (bf16, scaled e4m3)


@pytest.mark.parametrize("scaled", [0, 1])
@pytest.mark.parametrize("H", [1, 2, 4, 8, 16])
def test_pv_pass_asm_mfma_hazards(prefill_asm, H, scaled):
    name = [n for n in prefill_asm if f"prefill_bf16_kernelILi{H}ELi2ELb{scaled}E" in n]
    assert len(name) == 1
    bad = asm_hazards.violations(prefill_asm[name[0]])
    assert not bad, "\n".join(bad[:10])


def test_checker_catches_both_rules():
    """Planted sequences: an operand overwrite and an early accumulator copy."""
    war = [";;#ASMSTART", "s_nop 2", "v_mfma_f32_32x32x16_bf16 v[0:15], v[16:19], v[20:23], v[0:15]", ";;#ASMEND",
           "v_exp_f32_e32 v17, v30"]
    raw = [";;#ASMSTART", "v_mfma_f32_32x32x16_bf16 v[0:15], v[16:19], v[20:23], v[0:15]", ";;#ASMEND",
           "s_nop 7", "v_mov_b64_e32 v[40:41], v[2:3]"]
    ok = [";;#ASMSTART", "v_mfma_f32_32x32x16_bf16 v[0:15], v[16:19], v[20:23], v[0:15]",
          "s_nop 7", "s_nop 7", "s_nop 3", ";;#ASMEND", "v_exp_f32_e32 v17, v2"]
    assert len(asm_hazards.violations(war)) == 1
    assert len(asm_hazards.violations(raw)) == 1
    assert asm_hazards.violations(ok) == []
