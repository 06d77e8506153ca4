"""Oracle: slow, plain CPU definitions of every operation the library computes.

TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT. Only the tests, the smoke check
and the benchmark's CPU-baseline leg may import or call anything in this
package. It shares no code, tables, constants or helpers with the HIP library
(block_scaled_fp4_gemm_amd), and neither imports the other; both consume the
same seeded bytes from the standalone `synthetic` module.

Two independent implementations of the same definitions live here: the numpy
modules (codecs, gemm) and a plain C++17 one (cpu_oracle.cpp, built with
-O2 -ffp-contract=off and loaded through oracle.cpp). Each is pinned on its
own, and the two are compared with each other.

Every function is pinned by CPU tests against something other than itself
(textbook format tables, library dtype conversions, exact rational brute
force, closed-form identities and hand-worked rounding cases).
"""
from .codecs import (  # noqa: F401
    bf16_to_f32,
    bf16_to_f64,
    dequant_fp4,
    dequant_fp4_t,
    e2m1_to_f64,
    e4m3fn_to_f64,
    f32_to_bf16,
    scales_from_blocked,
    unpack_e2m1,
)
from .gemm import (  # noqa: F401
    gemm_bf16_ref,
    gemm_fp4_ref,
    gemm_fp4_splitk_planes_ref,
    gemm_ordered,
    gemm_ordered_f32,
    gemm_scaled_acc_exact,
    gemm_splitk_planes_ref,
    gemm_w4a16_exact,
    gemm_w4a16_ref,
    gemm_w4a16_t_ref,
    rms,
    scaled_acc_admissible,
    scaled_acc_candidate_deltas,
    scaled_acc_epilogue,
    splitk_chunk,
    splitk_reduce,
    tolerance,
)
