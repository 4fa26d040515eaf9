"""Host logic of bench.py's kernel roofline: the bound is the roof with the longer lower-bound time,
and the fraction is achieved over peak in that roof's unit (no GPU needed)."""
import bench


def test_hbm_roof_when_bytes_dominate():
    # 1.6 GB at 8 TB/s = 200 us against 0.7 TFLOP at 10.1 PFLOP/s = 69 us: HBM-bound
    r = bench.kernel_roof(1.6e9, 0.7e12, 10100.0, 400e-6)
    assert r["bound"] == "hbm" and r["unit"] == "GB/s"
    assert abs(r["achieved"] - 4000.0) < 0.1 and abs(r["frac"] - 0.5) < 1e-4
    assert abs(r["roof_us"]["hbm"] - 200.0) < 0.01 and abs(r["roof_us"]["mfma"] - 69.31) < 0.01


def test_mfma_roof_when_flops_dominate():
    # 0.722 TFLOP at 2.5 PFLOP/s = 289 us against 1.5 GB at 8 TB/s = 188 us: matrix-core bound
    r = bench.kernel_roof(1.5e9, 0.722e12, 2500.0, 578e-6)
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s" and r["peak"] == 2500.0
    assert abs(r["frac"] - 0.5) < 1e-3
    assert r["bytes_per_launch"] == 1500000000 and r["flops_per_launch"] == 722000000000


def test_tie_goes_to_hbm():
    r = bench.kernel_roof(8e9, 2.5e15 * 1e-3, 2500.0, 1e-3)   # both lower bounds are 1 ms
    assert r["bound"] == "hbm" and abs(r["frac"] - 1.0) < 1e-4
