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
    assert P.bench_name("__amd_rocclr_copyBuffer") is None
    assert P.source_hash("decode") != P.source_hash("prefill")


def test_missing_summary_gives_nothing(tmp_path):
    assert P.read_traffic(os.path.join(str(tmp_path), "absent.md")) == {}
