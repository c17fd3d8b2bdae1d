"""Host logic of the profile summaries: the benchmark takes a kernel's HBM
traffic only from a summary taken on that kernel path's current sources."""
import os

from quantized_moe_expert_gemv_amd import prof_summary as P


def _write(tmp_path, lines):
    p = os.path.join(tmp_path, "t.md")
    with open(p, "w") as f:
        f.write("\n".join(lines) + "\n")
    return p


def test_read_traffic_matches_path_sources(tmp_path):
    d, pf = P.source_hash("decode"), P.source_hash("prefill")
    p = _write(str(tmp_path), [
        "# header",
        f"traffic: kernel=gateup path=decode bytes_per_dispatch=100 sources={d}",
        f"traffic: kernel=down_combine path=decode bytes_per_dispatch=50 sources={'0' * 16}",
        f"traffic: kernel=gateup_gemm path=prefill bytes_per_dispatch=7 sources={pf}",
        "traffic: kernel=topk bytes_per_dispatch=3",
    ])
    assert P.read_traffic(p) == {"gateup": 100.0, "gateup_gemm": 7.0}


def test_kernel_paths_and_names():
    assert P.kernel_path("void strata::(anonymous namespace)::k_gateup<2, 4>(x)") == "decode"
    assert P.kernel_path("strata::(anonymous namespace)::k_gemm_gateup<2, false>(x)") == "prefill"
    assert P.bench_name("strata::(anonymous namespace)::k_down<2>(x)") == "down_combine"
    # the decode kernels of 9..16 tokens and the decode block top-k
    assert P.bench_name("void strata::(anonymous namespace)::k_down16<2, 7>(x)") == "down_combine"
    assert P.kernel_path("void strata::(anonymous namespace)::k_down16<2, 7>(x)") == "decode"
    assert P.bench_name("strata::(anonymous namespace)::k_topk_block_decode(x)") == "topk"
    assert P.kernel_path("strata::(anonymous namespace)::k_topk_block(x)") == "decode"   # built from decode.hip
    assert P.bench_name("__amd_rocclr_copyBuffer") is None
    assert P.source_hash("decode") != P.source_hash("prefill")


def test_missing_summary_gives_nothing(tmp_path):
    assert P.read_traffic(os.path.join(str(tmp_path), "absent.md")) == {}


def test_read_mfma_matches_path_sources(tmp_path):
    pf = P.source_hash("prefill")
    p = _write(str(tmp_path), [
        f"mfma: kernel=gateup_gemm path=prefill busy_frac=0.5 mfma_flops=1000 valu_per_mfma=1.5 sources={pf}",
        f"mfma: kernel=down_gemm path=prefill busy_frac=0.4 mfma_flops=10 valu_per_mfma=1 sources={'0' * 16}",
    ])
    assert P.read_mfma(p) == {"gateup_gemm": {"busy_frac": 0.5, "mfma_flops": 1000.0, "valu_per_mfma": 1.5}}


def test_mfma_summary_from_counter_rows(tmp_path):
    """The busy fraction divides the summed MFMA busy cycles by the cycles of
    every SIMD of the device (GRBM_GUI_ACTIVE is summed over the 8 dies)."""
    import csv
    rows = []
    kern = "void strata::(anonymous namespace)::k_gemm_gateup<2, 4>(x)"
    for d in range(2):
        for name, val in (("SQ_VALU_MFMA_BUSY_CYCLES", 0.5 * 1000 * 4 * 256), ("SQ_INSTS_MFMA", 100.0),
                          ("SQ_INSTS_VALU", 250.0), ("SQ_INSTS_VALU_MFMA_MOPS_F16", 32.0),
                          ("GRBM_GUI_ACTIVE", 8 * 1000.0)):
            rows.append({"Kernel_Name": kern, "Counter_Name": name, "Counter_Value": val})
    src = os.path.join(str(tmp_path), "pmc.csv")
    with open(src, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        w.writerows(rows)
    out = os.path.join(str(tmp_path), "m.md")
    P.mfma(out, "cmd", src, 256)
    got = P.read_mfma(out)["gateup_gemm"]
    assert abs(got["busy_frac"] - 0.5) < 1e-9
    assert got["mfma_flops"] == 32 * 512
    assert abs(got["valu_per_mfma"] - 1.5) < 1e-9
