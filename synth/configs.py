"""The five synthetic workloads: shapes, value distributions, mode and scalar parameters.

Modes: "int32" = per-token int4 packed 8 per int32 word [K, M, N/8]; "int4" = per-token
int4 packed 2 per byte [K, M, N]; "fp4" = per-group-32 E2M1 [K, M*N] with e8m0 scales
[K, ceilDiv(M*N, 64), 2]; "int8" / "e4m3" / "e5m2" = per-token 8-bit codes [K, M, N].
The next five run the 64 x 64 and the two-sided 256 x 256 activation workloads with 8-bit
codes; the last has a side above 128.  Transform matrices are Haar-random orthogonal matrices rounded
to the activation dtype; ``two_sided=False`` passes an empty [0, 0] right transform.
"""
from __future__ import annotations

from dataclasses import dataclass, replace


@dataclass(frozen=True)
class Workload:
    name: str
    K: int
    M: int
    N: int
    dtype: str            # "bf16" | "f16"
    dist: str             # "gauss" | "laplace"
    outlier_frac: float
    outlier_scale: float
    mode: str             # "int32" | "int4" | "fp4"
    clip_ratio: float
    dst_type_max: float
    two_sided: bool = True
    seed: int = 0

    @property
    def elems(self) -> int:
        return self.K * self.M * self.N

    def with_K(self, K: int) -> "Workload":
        return replace(self, K=K)


WORKLOADS = {
    "c1": Workload("K64_M16_N16_bf16_int32_clip1.0", 64, 16, 16, "bf16", "gauss", 0.0, 1.0,
                   "int32", 1.0, 0.0),
    "c2": Workload("K8192_M64_N64_bf16_out1pct_x20_int32_clip0.9", 8192, 64, 64, "bf16", "gauss",
                   0.01, 20.0, "int32", 0.9, 0.0),
    "c3": Workload("K16384_M64_N128_f16_out0.5pct_x50_mxfp4_v1", 16384, 64, 128, "f16", "gauss",
                   0.005, 50.0, "fp4", 1.0, 0.0),
    "c4": Workload("K32768_M256_N256_bf16_out1pct_x20_int4_clip0.95", 32768, 256, 256, "bf16",
                   "gauss", 0.01, 20.0, "int4", 0.95, 0.0),
    "c5": Workload("K16384_M256_N256_bf16_laplace_out1pct_x30_leftonly_mxfp4_v2_dmax8", 16384, 256,
                   256, "bf16", "laplace", 0.01, 30.0, "fp4", 1.0, 8.0, two_sided=False),
    "c2i8": Workload("K8192_M64_N64_bf16_out1pct_x20_int8_clip1.0", 8192, 64, 64, "bf16", "gauss",
                     0.01, 20.0, "int8", 1.0, 0.0),
    "c2e4m3": Workload("K8192_M64_N64_bf16_out1pct_x20_fp8e4m3_clip1.0", 8192, 64, 64, "bf16", "gauss",
                       0.01, 20.0, "e4m3", 1.0, 0.0),
    "c2e5m2": Workload("K8192_M64_N64_bf16_out1pct_x20_fp8e5m2_clip1.0", 8192, 64, 64, "bf16", "gauss",
                       0.01, 20.0, "e5m2", 1.0, 0.0),
    "c4i8": Workload("K32768_M256_N256_bf16_out1pct_x20_int8_clip1.0", 32768, 256, 256, "bf16",
                     "gauss", 0.01, 20.0, "int8", 1.0, 0.0),
    "c4e4m3": Workload("K32768_M256_N256_bf16_out1pct_x20_fp8e4m3_clip1.0", 32768, 256, 256, "bf16",
                       "gauss", 0.01, 20.0, "e4m3", 1.0, 0.0),
    # a side above 128: hidden 28672 as 224 x 128 (the MLP width of a 70B-class model), which
    # runs padded to 256 x 256
    "p224": Workload("K16384_M224_N128_bf16_out1pct_x20_int32_clip0.9", 16384, 224, 128, "bf16", "gauss",
                     0.01, 20.0, "int32", 0.9, 0.0),
}
