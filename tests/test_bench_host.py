"""bench.py's host-side choices (no GPU): which expert kernels a workload's launches run,
and where the benchmark packs the expert weights, following the library's rules (the
library's bound on the kept rows per expert: >= 256 the packed-weight kernel, < 48 the
32-row tiles, float32 the SIMT kernel)."""
import bench
from sparse_mixture_experts_forward_amd import CONFIGS
from sparse_mixture_experts_forward_amd import _binding as B


def _cap(c):
    return B.moe_capacity_rule(c.n_tokens, c.n_experts, c.top_k, B.CAPACITY_RULES[c.capacity_rule],
                               c.alpha or 0.0)


def test_stage_kernels_of_the_workloads():
    want = {  # workload: (packed?, gemm1 kernel, gemm2 kernel) with packing allowed
        "mixtral": (True, "gemm_packed_kernel<2>", "gemm_packed_kernel<0>"),
        "decode": (True, "gemm_packed_small_kernel<2>", "gemm_packed_small_kernel<0>"),
        "deepseek": (False, "gemm_bf16_kernel<256, 2, false>", "gemm_bf16_kernel<256, 0, false>"),
        "switch": (False, "gemm_bf16_kernel<256, 1, false>", "gemm_bf16_kernel<256, 0, false>"),
        "tiny": (False, "gemm_f32_kernel<1, false>", "gemm_f32_kernel<0, false>"),
    }
    for name, (packed, k1, k2) in want.items():
        c = CONFIGS[name]
        cap = _cap(c)
        pk = bench.packed_path(c, cap, True)
        assert pk == packed, name
        assert bench.stage_symbol(c, "gemm1", pk, cap) == k1, name
        assert bench.stage_symbol(c, "gemm2", pk, cap) == k2, name
        assert bench.stage_symbol(c, "route", pk, cap) is None
        assert not bench.packed_path(c, cap, False)


def test_kernel_rules_at_the_thresholds():
    m = CONFIGS["mixtral"]
    # 256 rows per expert (N k / E): packed kernel; 255: staged 256-row tiles; 47: 32-row
    for n, packed, k1 in ((1024, True, "gemm_packed_kernel<2>"),
                          (1020, False, "gemm_bf16_kernel<256, 2, false>"),
                          (188, True, "gemm_packed_small_kernel<2>")):
        c = m.with_tokens(n)
        assert bench.packed_path(c, -1, True) == packed, n
        assert bench.stage_symbol(c, "gemm1", packed, -1) == k1, n
    assert bench.stage_symbol(m.with_tokens(188), "gemm1", False, -1) == "gemm_bf16_kernel<32, 2, false>"
    # a capacity bounds the rows: 4096 tokens, capacity 20 -> 20 rows per expert
    assert bench.stage_symbol(m, "gemm2", True, 20) == "gemm_packed_small_kernel<0>"
