"""Checks on the gfx950 machine code of the HIP kernels (CPU only: hipcc cross-compiles).

On gfx950, a 16x16x16 MFMA that takes as its accumulator input the result of a 16x16x32 MFMA
(a "mixed-shape accumulator chain") was measured to read a stale accumulator: results were wrong
in a way that depended on the instruction schedule. The kernels therefore keep terms of different
MFMA shapes in separate accumulators. This test compiles every kernel source to gfx950 assembly
with the library's own flags and fails if any such chain appears in the generated code.
"""
import os
import re
import shutil
import subprocess

import pytest

from test_sequence_layers_amd import build as B

HIPCC = B.HIPCC if os.path.exists(B.HIPCC) else shutil.which("hipcc")
KERNEL_SOURCES = [s for s in B.SOURCES if s != "abi.hip"]


def _regs(tok):
    tok = tok.strip()
    m = re.match(r"([va])\[(\d+):(\d+)\]$", tok)
    if m:
        return {(m.group(1), r) for r in range(int(m.group(2)), int(m.group(3)) + 1)}
    m = re.match(r"([va])(\d+)$", tok)
    return {(m.group(1), int(m.group(2)))} if m else set()


def mixed_shape_chains(asm_lines):
    """(distance, producer, consumer) for every MFMA whose accumulator input (SrcC) was last
    written by an MFMA of a different opcode within the same basic block."""
    ins = [ln.strip() for ln in asm_lines]
    ins = [ln for ln in ins if ln and not ln.startswith((";", "."))]
    hits = []
    for i, line in enumerate(ins):
        if not line.startswith("v_mfma"):
            continue
        op, rest = line.split(None, 1)
        ops = [t.strip() for t in rest.split(",")]
        if len(ops) < 4:
            continue
        src_c = _regs(ops[3])
        if not src_c:
            continue
        for j in range(i - 1, -1, -1):
            prev = ins[j]
            if prev.endswith(":") or prev.startswith(("s_cbranch", "s_branch", "s_barrier", "s_setpc")):
                break
            if " " not in prev:
                continue
            pop, prest = prev.split(None, 1)
            if pop.startswith(("ds_write", "global_store", "buffer_store", "scratch_store", "s_")):
                continue
            if _regs(prest.split(",")[0]) & src_c:
                if pop.startswith("v_mfma") and pop != op:
                    hits.append((i - j, pop, op))
                break
    return hits


def test_scanner_finds_a_planted_chain():
    planted = [
        "v_mfma_f32_16x16x32_bf16 v[10:13], v[0:3], v[4:7], 0",
        "v_cvt_pk_bf16_f32 v20, v21, v22",
        "v_mfma_f32_16x16x16_bf16 v[10:13], v[14:15], v[16:17], v[10:13]",
        "v_mov_b32_e32 v30, 0",
        "v_mfma_f32_16x16x32_bf16 v[40:43], v[0:3], v[4:7], 0",
        "v_mov_b32_e32 v40, 0",  # an intervening write breaks the dependency
        "v_mfma_f32_16x16x16_bf16 v[40:43], v[14:15], v[16:17], v[40:43]",
    ]
    assert mixed_shape_chains(planted) == [(2, "v_mfma_f32_16x16x32_bf16", "v_mfma_f32_16x16x16_bf16")]


@pytest.mark.skipif(HIPCC is None, reason="hipcc not available")
@pytest.mark.parametrize("src", KERNEL_SOURCES)
def test_no_mixed_shape_mfma_accumulator_chains(src, tmp_path):
    out = tmp_path / (src + ".s")
    cmd = [HIPCC, *[f for f in B.flags_for(src) if f != "-fPIC"], "--cuda-device-only", "-S",
           os.path.join(B.CSRC, src), "-o", str(out)]
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert p.returncode == 0, p.stdout[-2000:]
    hits = mixed_shape_chains(out.read_text().splitlines())
    assert not hits, f"{src}: mixed-shape MFMA accumulator chains {hits[:5]}"


def _mlp_erf_coefficients():
    src = open(os.path.join(B.CSRC, "mlp.hip")).read()
    m = re.search(r"kErfP\[(\d+)\]\s*=\s*\{([^}]*)\}", src)
    assert m, "kErfP not found in mlp.hip"
    coef = [float(x.strip().rstrip("f")) for x in m.group(2).split(",")]
    assert len(coef) == int(m.group(1))
    return coef


def test_mlp_fast_gelu_polynomial_matches_erf():
    """The TTT-MLP kernel's fast GELU path evaluates erf(u) = u P(u^2) for |u| <= 1 and
    Phi(x) = 1/2 + x R(x^2) for x^2 <= 2, R(t) = P(t / 2) / (2 sqrt 2). Evaluated here in fp32
    Horner form with the kernel's own coefficients, both stay within 3e-5 of scipy's erf / normal
    CDF (the products that consume GELU's output round their operands to bf16, 3.9e-3)."""
    import numpy as np
    from scipy.special import erf, ndtr

    p = [np.float32(c) for c in _mlp_erf_coefficients()]
    u = np.linspace(-1.0, 1.0, 400001).astype(np.float32)
    s = u * u
    acc = p[-1]
    for c in p[-2::-1]:
        acc = acc * s + c
    assert np.abs((u * acc).astype(np.float64) - erf(u.astype(np.float64))).max() < 3e-5
    k = np.float32(0.35355339059327376220)
    r = [np.float32(p[i] * k / np.float32(2 ** i)) for i in range(len(p))]
    x = np.linspace(-np.sqrt(2.0), np.sqrt(2.0), 400001).astype(np.float32)
    t = x * x
    acc = r[-1]
    for c in r[-2::-1]:
        acc = acc * t + c
    cdf = x * acc + np.float32(0.5)
    assert np.abs(cdf.astype(np.float64) - ndtr(x.astype(np.float64))).max() < 3e-5


def _mlp_slope_coefficients():
    src = open(os.path.join(B.CSRC, "mlp.hip")).read()
    coef = {int(m.group(1)): float(m.group(2)) for m in re.finditer(r"kS(\d)\s*=\s*([-+0-9.eE]+)f", src)}
    assert sorted(coef) == [0, 1, 2, 3], "kS0..kS3 not found in mlp.hip"
    return [coef[i] for i in range(4)]


def test_mlp_fast_gelu_in_fp16():
    """The fast path runs in packed fp16: Phi(x) = 1/2 + x R(t), GELU(x) = x Phi(x) and
    GELU'(x) = 1/2 + x S(t), t = x^2 <= 2, Horner form, every operation rounded to fp16 (numpy
    rounds the product and the sum of each step separately, one rounding more than the hardware's
    fused multiply-add). GELU and GELU' stay within 1.5e-3 of the exact values over |x| <= sqrt 2,
    about the rounding of a bf16 operand of that size."""
    import numpy as np
    from scipy.special import ndtr

    h = np.float16
    k = 0.35355339059327376220
    r = [np.float32(c * k / 2 ** i) for i, c in enumerate(_mlp_erf_coefficients())]
    s = _mlp_slope_coefficients()
    x = np.linspace(-np.sqrt(2.0), np.sqrt(2.0), 400001).astype(h)
    t = (x * x).astype(h)

    def horner(cs):
        acc = h(cs[-1])
        for c in cs[-2::-1]:
            acc = (acc * t).astype(h)
            acc = (acc + h(c)).astype(h)
        return acc

    cdf = ((x * horner(r)).astype(h) + h(0.5)).astype(h)
    gelu = (x * cdf).astype(h).astype(np.float64)
    slope = ((x * horner(s)).astype(h) + h(0.5)).astype(h).astype(np.float64)
    xd = x.astype(np.float64)
    phi = np.exp(-xd * xd / 2) / np.sqrt(2 * np.pi)
    assert np.abs(gelu - xd * ndtr(xd)).max() < 1.5e-3
    assert np.abs(slope - (ndtr(xd) + xd * phi)).max() < 1.5e-3



def _occ_table(src, name):
    m = re.search(name + r"\[3\]\[3\]\[2\]\s*=\s*\{(.*?)\};", src, flags=re.S)
    assert m, f"{name} not found"
    body = re.sub(r"//[^\n]*", "", m.group(1))
    vals = [int(x) for x in re.findall(r"\d+", body)]
    assert len(vals) == 18
    return {(d, c, b): vals[(i * 3 + j) * 2 + b] for i, d in enumerate((16, 32, 64)) for j, c in enumerate((16, 32, 64))
            for b in (0, 1)}


@pytest.mark.skipif(HIPCC is None, reason="hipcc not available")
def test_chunk_plan_occupancy_tables_match_the_compiled_kernels(tmp_path):
    """The chunked scans size their segment plan from fixed tables of the waves per SIMD that each
    compiled compose / scan kernel sustains (so that the plan does not depend on the device a call
    runs on). Those tables must equal the compiler's occupancy report for the current sources. The
    column-order instances of the bidirectional kernels (the 2-D scan) run on the same plan, so they
    must keep at least the plan's workgroups per CU resident (both kernels have D / 16 waves per
    workgroup; the plan takes the smaller figure of compose and scan, at most 12 waves per CU)."""
    src_path = os.path.join(B.CSRC, "chunked.hip")
    src = open(src_path).read()
    compose, scan = _occ_table(src, "kComposeOcc"), _occ_table(src, "kScanOcc")
    cmd = [HIPCC, *[f for f in B.flags_for("chunked.hip") if f != "-fPIC"], "--cuda-device-only", "-c", src_path,
           "-o", str(tmp_path / "c.o"), "-Rpass-analysis=kernel-resource-usage"]
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert p.returncode == 0, p.stdout[-2000:]
    found, cols = {}, {}
    kernel = None
    for line in p.stdout.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            kernel = m.group(1)
            continue
        m = re.search(r"Occupancy \[waves/SIMD\]: (\d+)", line)
        if m and kernel:
            k = re.search(r"(chunk_compose_bf16|chunk_scan_bf16)ILi(\d+)ELi(\d+)EL([bi])(\d)E(Lb1E)?", kernel)
            if k:
                key = (k.group(1), int(k.group(2)), int(k.group(3)), int(k.group(5)))
                (cols if k.group(6) else found)[key] = int(m.group(1))
    assert len(found) == 36, sorted(found)
    assert len(cols) == 18 and all(key[3] == 1 for key in cols), sorted(cols)
    for (kind, d, c, bidir), occ in found.items():
        table = compose if kind == "chunk_compose_bf16" else scan
        assert table[(d, c, bidir)] == occ, f"{kind}<{d}, {c}, {'bidir' if bidir else 'causal'}>: table " \
                                             f"{table[(d, c, bidir)]}, compiler {occ}"
    waves_per_cu = int(re.search(r"kPlanWavesPerCU = (\d+);", src).group(1))
    max_groups = int(re.search(r"kMaxGroupsPerCU = (\d+);", src).group(1))

    def plan_groups(d, c, bidir):
        w = d // 16
        n = min(4 * compose[(d, c, bidir)] // w, 4 * scan[(d, c, bidir)] // w, waves_per_cu // w)
        return max(1, min(max_groups, n))

    for (kind, d, c, bidir), occ in cols.items():
        need = plan_groups(d, c, bidir)
        assert 4 * occ // (d // 16) >= need, f"{kind}<{d}, {c}, bidir, column order>: {occ} waves per SIMD " \
                                             f"keep fewer than the plan's {need} workgroups per CU"


def _mlp_as_constants():
    src = open(os.path.join(B.CSRC, "mlp.hip")).read()
    names = ["kAsP", "kAsA1", "kAsA2", "kAsA3", "kAsA4", "kAsA5"]
    vals = {n: float(m.group(1)) for n in names for m in [re.search(n + r"\s*=\s*([-+0-9.eE]+)f", src)] if m}
    assert sorted(vals) == sorted(names), "Abramowitz-Stegun constants not found in mlp.hip"
    return [vals[n] for n in names]


def test_mlp_wide_gelu_erf_approximation():
    """The wide TTT-MLP kernel's GELU and GELU' (cdf_as): erf by Abramowitz and Stegun 7.1.26 with the
    kernel's constants, in fp32 like the kernel (exp2 and the reciprocal rounded to fp32), against
    scipy's normal CDF and density: GELU within 3e-7 relative to max(1, |x|), GELU' within 3e-7,
    over |x| <= 12 (the published bound on erf is 1.5e-7)."""
    import numpy as np
    from scipy.special import ndtr

    p, a1, a2, a3, a4, a5 = [np.float32(c) for c in _mlp_as_constants()]
    f = np.float32
    x = np.linspace(-12.0, 12.0, 2000001).astype(f)
    e = np.exp2(x * x * f(-0.72134752044448170368)).astype(f)
    t = (f(1) / (p * (np.abs(x) * f(0.70710678118654752440)) + f(1))).astype(f)
    poly = t * (a1 + t * (a2 + t * (a3 + t * (a4 + t * a5))))
    cdf = (f(0.5) + np.copysign(f(0.5) * (f(1) - poly * e), x)).astype(f)
    gelu = (x * cdf).astype(np.float64)
    slope = (x * e * f(0.39894228040143267794) + cdf).astype(np.float64)
    xd = x.astype(np.float64)
    phi = np.exp(-xd * xd / 2) / np.sqrt(2 * np.pi)
    assert np.max(np.abs(gelu - xd * ndtr(xd)) / np.maximum(1.0, np.abs(xd))) < 3e-7
    assert np.max(np.abs(slope - (ndtr(xd) + xd * phi))) < 3e-7
