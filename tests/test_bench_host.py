"""bench.py's host-side choices (no GPU): which expert kernels a workload's launches run,
and where the benchmark packs the expert weights, following the library's rules (with
packed weights, by the library's bound on the kept rows per expert: >= 256 the 128 x 512
shape, 48 .. 255 the 256 x 256 shape, < 48 the 32-row kernel; staged weights: >= 48 the
256-row tiles, < 48 the 32-row tiles; float32 the SIMT kernel, on 32 x 32 tiles where
64 x 64 tiles would number under 512)."""
import bench
from sparse_mixture_experts_forward_amd import CONFIGS
from sparse_mixture_experts_forward_amd import _binding as B


def _cap(c):
    return B.moe_capacity_rule(c.n_tokens, c.n_experts, c.top_k, B.CAPACITY_RULES[c.capacity_rule],
                               c.alpha or 0.0)


def test_stage_kernels_of_the_workloads():
    want = {  # workload: (packed?, gemm1 kernel, gemm2 kernel) with packing allowed
        "mixtral": (True, "gemm_packed_kernel<PackedShape<128, 8, 8, 0>, 2>", "gemm_packed_kernel<PackedShape<128, 8, 8, 0>, 0>"),
        "decode": (True, "gemm_packed_small_kernel<2>", "gemm_packed_small_kernel<0>"),
        "deepseek": (True, "gemm_packed_kernel<PackedShape<256, 16, 4, 1>, 2>", "gemm_packed_kernel<PackedShape<256, 16, 4, 1>, 0>"),
        "switch": (True, "gemm_packed_kernel<PackedShape<256, 16, 4, 1>, 1>", "gemm_packed_kernel<PackedShape<256, 16, 4, 1>, 0>"),
        "tiny": (False, "gemm_f32_kernel<1, false, 32>", "gemm_f32_kernel<0, false, 32>"),
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
    # 256 rows per expert (N k / E): 128 x 512 kernel; 255: mid-size; 47: 32-row
    for n, k1, staged in ((1024, "gemm_packed_kernel<PackedShape<128, 8, 8, 0>, 2>", "gemm_bf16_kernel<256, 2, false>"),
                          (1020, "gemm_packed_kernel<PackedShape<256, 16, 4, 1>, 2>", "gemm_bf16_kernel<256, 2, false>"),
                          (192, "gemm_packed_kernel<PackedShape<256, 16, 4, 1>, 2>", "gemm_bf16_kernel<256, 2, false>"),
                          (188, "gemm_packed_small_kernel<2>", "gemm_bf16_kernel<32, 2, false>")):
        c = m.with_tokens(n)
        assert bench.packed_path(c, -1, True), n
        assert bench.stage_symbol(c, "gemm1", True, -1) == k1, n
        assert bench.stage_symbol(c, "gemm1", False, -1) == staged, n
    # a capacity bounds the rows: 4096 tokens, capacity 20 -> 20 rows per expert
    assert bench.stage_symbol(m, "gemm2", True, 20) == "gemm_packed_small_kernel<0>"


def test_float32_tile_choice():
    t = CONFIGS["tiny"]
    # 512 rows over 8 experts: 64 x 64 tiles number (8 + 8) x 8 = 128 (gemm1), x 2 (gemm2)
    assert bench._f32_tile(t, "gemm1", -1) == 32 and bench._f32_tile(t, "gemm2", -1) == 32
    big = t.with_tokens(8192)  # (256 + 8) x 8 = 2112 tiles of 64 x 64 for gemm1
    assert bench._f32_tile(big, "gemm1", -1) == 64
