"""The profile summaries' kernel classes (CPU): every decode-step kernel
name, with or without the GEMV's optional row-tiles argument and for the
staged and the chunk-streamed GEMV items, lands in the class the summaries
report it under."""
from paged_kv_gqa_qwen3_amd import rocprof_summary as rs


def test_kernel_classes():
    cases = {
        "void qd::gemv_kernel<8, 4>(qd::GemvArgs)": "qkv",
        "void qd::gemv_kernel<16, 4, 1>(qd::GemvArgs)": "qkv",
        "void qd::gemv_kernel<16, 2, 2>(qd::GemvArgs)": "gate_up",
        "void qd::gemv_kernel<16, 1, 2>(qd::GemvArgs)": "o_proj+down",
        "void qd::gemv_kernel<16, 3, 2>(qd::GemvArgs)": "lm_head",
        "void qd::gemv_kernel<1, 3>(qd::GemvArgs)": "lm_head",
        "void qd::gemv_wide_kernel<16, 3, 2>(qd::GemvArgs)": "lm_head",
        "void qd::gemv_wide_kernel<64, 1, 2>(qd::GemvArgs)": "o_proj+down",
        "void qd::gemv_wide_kernel<32, 4, 2>(qd::GemvArgs)": "qkv",
        "void qd::fused_mlp_kernel<16, 2, 1>(qd::FusedMlpArgs)": "gate_up+down",
        "void qd::attention_kernel<128, 4, 8, 3, qd::KvBf16>(qd::AttnArgs)": "attention",
        "void qd::stream_step_kernel<128, 4>(qd::StreamArgs)": "stream_step",
        "qd::sample_kernel(qd::SampleArgs)": "sample",
        "qd::sample_sum_kernel(qd::SampleArgs)": "sample_sum",
        "qd::sample_nucleus_kernel(qd::SampleArgs)": "sample_nucleus",
        "void qd::pf_gemm_kernel<2, 4, 2, 8>(qd::PfGemmArgs)": "pf_gate_up",
        "qd::repack_kernel(unsigned short const*, int, int, unsigned short*, int, int, int)": None,
    }
    for name, cls in cases.items():
        assert rs.kernel_class(name) == cls, name
