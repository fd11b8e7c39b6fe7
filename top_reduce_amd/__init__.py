"""top_reduce_amd: one GPU's share of an expert-parallel MoE FFN on MI355X.

Route scan -> expand -> grouped SwiGLU GEMM -> weighted top-k reduce, as
hand-written gfx950 HIP kernels behind the C ABI of ``libtopreduce.so``
(``include/topreduce.h``). This package is the thin Python binding: it checks
and marshals PyTorch tensors (device memory and streams only) and calls the
library; every step of the path runs in the library's kernels. There is no
fallback: if the library is not built, importing the binding's entry points
raises.

Entry points: ``plan`` (route scan; with ``block_rows``/``block_counts`` over
a DP-padded buffer), ``forward`` (the whole layer), the stages ``expand``,
``grouped_gemm`` (``grouped_gemm_up``/``_down``, ``grouped_gemm_up_x``
gathering x, ``grouped_gemm_down_y`` writing single-slot rows to y),
``combine_reduce`` / ``combine_reduce_multi``, the cross-rank
``combine_epilogue``, ``compact_rows`` (effective rows of a padded buffer)
and ``plan_stats``. ``FLAG_NO_XE`` plans without the expanded-row buffer.
``forward_noalloc`` is plan + forward in the library's own static workspace,
for callers that cannot allocate device memory.
"""

from ._binding import (  # noqa: F401
    ABI_VERSION,
    BF16,
    F32,
    FLAG_GEMM_FORCE_STREAM,
    FLAG_GEMM_FORCE_TILED,
    FLAG_NO_XE,
    NOALLOC_SCRATCH_BYTES,
    MoePlan,
    TopReduceError,
    combine_epilogue,
    compact_rows,
    combine_reduce,
    combine_reduce_multi,
    expand,
    forward,
    forward_noalloc,
    grouped_gemm,
    grouped_gemm_down,
    grouped_gemm_down_y,
    grouped_gemm_up,
    grouped_gemm_up_x,
    lib_path,
    load_library,
    make_desc,
    plan,
    plan_stats,
    workspace_size,
)
