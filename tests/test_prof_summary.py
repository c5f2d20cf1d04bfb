"""Host logic of the profile summaries: the source hash that marks recorded
HBM counters stale, and the kernel roles read from demangled names."""
from sparse_mixture_experts_scan_amd import prof_summary as P


def test_code_text_ignores_comments_and_whitespace():
    a = "int f(int x) {  // doubles\n  return 2 * x; /* no overflow\n check */ }\n"
    b = "int f(int x) {\n\n    return 2 * x;\n}"
    assert P.code_text(a) == P.code_text(b) == "int f(int x) { return 2 * x; }"
    # a change to the code itself changes the text
    assert P.code_text(a.replace("2 * x", "3 * x")) != P.code_text(a)


def test_kernel_roles():
    assert P.kernel_key("void moe::stream_dma_kernel<16, 16, true>(unsigned short const*)") == "gateup"
    assert P.kernel_key("void moe::stream_dma_kernel<16, 16, false>(unsigned short const*)") == "down"
    assert P.kernel_key("void moe::tile_gemm_kernel<true>(unsigned short const*)") == "gateup"
    assert P.kernel_key("void moe::tile_gemm_kernel<false>(unsigned short const*)") == "down"
    assert P.kernel_key("void moe::stream_q4_dma_kernel<16, 32, true>(unsigned short const*)") == "gateup"
    assert P.kernel_key("void moe::stream_q4_dma_kernel<16, 64, false>(unsigned short const*)") == "down"
