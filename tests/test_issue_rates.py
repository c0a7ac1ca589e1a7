"""Host logic of the VALU roofline basis (weight_decompression_amd/issue_rates.py): the
counter category of each timed instruction read from rocprofv3 CSV output, the static
assembly mix of one kernel, and the dynamic-mix peak N / sum_c(N_c / r_c)."""

import collections
import csv
import os

import pytest

from weight_decompression_amd import issue_rates as ir


def _write_pmc(path, rows):
    os.makedirs(path, exist_ok=True)
    with open(os.path.join(path, "pmc_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for r in rows:
            w.writerow(r)


def test_categories_from_counter_runs(tmp_path):
    iters = 8192
    grid = 1024 * 256
    timed = grid / 64 * iters
    a, b = str(tmp_path / "a"), str(tmp_path / "b")
    _write_pmc(a, [
        {"Kernel_Name": "k_add_u32(unsigned int*, unsigned int)", "Grid_Size": grid,
         "Counter_Name": "SQ_INSTS_VALU_INT32", "Counter_Value": timed * 1.02},
        {"Kernel_Name": "k_add_u32(unsigned int*, unsigned int)", "Grid_Size": grid,
         "Counter_Name": "SQ_INSTS_VALU_INT32", "Counter_Value": timed * 1.00},   # second dispatch: mean
        {"Kernel_Name": "k_perm_b32(unsigned int*, unsigned int)", "Grid_Size": grid,
         "Counter_Name": "SQ_INSTS_VALU_INT32", "Counter_Value": timed * 0.01},
        {"Kernel_Name": "k_fma_f64(unsigned int*, unsigned int)", "Grid_Size": grid,
         "Counter_Name": "SQ_INSTS_VALU_FMA_F64", "Counter_Value": timed},
    ])
    _write_pmc(b, [
        {"Kernel_Name": "k_mul_f32(unsigned int*, unsigned int)", "Grid_Size": grid,
         "Counter_Name": "SQ_INSTS_VALU_MUL_F32", "Counter_Value": timed * 0.999},
    ])
    cats = ir.categories([a, b], iters)
    assert cats["v_add_u32"][0] == "SQ_INSTS_VALU_INT32" and cats["v_add_u32"][1] == pytest.approx(1.01)
    assert cats["v_perm_b32"][0] == ir.OTHER
    assert cats["v_fma_f64"][0] == "SQ_INSTS_VALU_FMA_F64"
    assert cats["v_mul_f32"][0] == "SQ_INSTS_VALU_MUL_F32"
    assert "v_sub_u32" not in cats
    # aliases inherit the category of the instruction they are timed as
    assert ir.category_of("v_cmp_gt_i32", {"v_cmp_ne_u32": (ir.OTHER, 0.0)}) == ir.OTHER


def test_mix_peak_is_the_harmonic_mix_of_categories():
    rates = {"v_add_u32": 1.4, "v_mad_u32_u24": 0.8, "v_fma_f64": 0.7, "v_perm_b32": 0.9, "v_mov_b32": 1.5}
    cats = {"v_add_u32": ("SQ_INSTS_VALU_INT32", 1.0), "v_mad_u32_u24": ("SQ_INSTS_VALU_INT32", 1.0),
            "v_fma_f64": ("SQ_INSTS_VALU_FMA_F64", 1.0), "v_perm_b32": (ir.OTHER, 0.0),
            "v_mov_b32": (ir.OTHER, 0.0)}
    static = collections.Counter({"v_add_u32": 30, "v_mad_u32_u24": 10, "v_fma_f64": 5, "v_perm_b32": 20,
                                  "v_mfma_f32_16x16x32_bf16": 4, "v_unknown_op": 3})
    dyn = {"SQ_INSTS_VALU": 1000.0 + 50.0, "SQ_INSTS_MFMA": 50.0, "SQ_INSTS_VALU_INT32": 600.0,
           "SQ_INSTS_VALU_FMA_F64": 100.0}
    rate, table, unplaced = ir.mix_peak(dyn, static, rates, cats)
    r_int = 40 / (30 / 1.4 + 10 / 0.8)
    want = 1000.0 / (600 / r_int + 100 / 0.7 + 300 / 0.9)
    assert rate == pytest.approx(want, rel=1e-12)
    rows = {c: (n, r) for c, n, r, _ in table}
    assert rows[ir.OTHER][0] == pytest.approx(300.0)
    assert rows["SQ_INSTS_VALU_INT32"][1] == pytest.approx(r_int)
    assert unplaced == collections.Counter({"v_unknown_op": 3})
    # a category executed but absent from the assembly falls back to the slowest measured rate
    dyn2 = dict(dyn, SQ_INSTS_VALU_TRANS_F64=100.0)
    rate2, _, _ = ir.mix_peak(dyn2, static, rates, cats)
    assert rate2 == pytest.approx(1000.0 / (600 / r_int + 100 / 0.7 + 100 / 0.7 + 200 / 0.9), rel=1e-12)


def test_rates_table_round_trip(tmp_path):
    rates = {n: 0.5 + i / 100 for i, n in enumerate(ir.NAMES)}
    cats = {n: ("SQ_INSTS_VALU_INT32" if i % 2 else ir.OTHER, 0.25 * (i % 5)) for i, n in enumerate(ir.NAMES)}
    p = tmp_path / "rates.md"
    p.write_text(ir.rates_table(rates, cats) + "\n")
    r2, c2 = ir.read_rates_md(str(p))
    assert r2 == pytest.approx(rates, abs=5e-4)
    assert {k: v[0] for k, v in c2.items()} == {k: v[0] for k, v in cats.items()}


def test_kernel_mix_counts_one_function(tmp_path):
    s = tmp_path / "k.s"
    s.write_text("\n".join([
        "_Z3fooPi:", "  v_add_u32_e32 v0, v1, v2", "  v_perm_b32 v0, v1, v2, v3", "  s_endpgm",
        "_Z3barPi:", "  v_add_u32_e32 v0, v1, v2", "  v_add_u32_e64 v0, v1, v2", "  v_cmp_ne_u32_e32 vcc, v0, v1",
        "  s_endpgm"]) + "\n")
    assert ir.kernel_mix(str(s), "3bar") == collections.Counter({"v_add_u32": 2, "v_cmp_ne_u32": 1})
