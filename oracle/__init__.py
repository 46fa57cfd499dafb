"""CPU oracle for paged-KV decode attention (float64, numpy).

TEST INFRASTRUCTURE. The oracle defines what the GPU path must compute and
is used only to check it: the tests, the smoke check and the benchmark's
CPU-baseline leg may import it; the library under
``paged_kv_attention_14_amd`` never does, and the oracle never imports that
library. The two share no code; only the seeded input generator in
``workloads`` feeds both.

Every function here is pinned by ``tests/test_oracle_*.py`` to something
other than itself: torch's fp64 scaled-dot-product attention on contiguous
K/V, scalar brute force with ``math.fsum``, closed forms (single token,
identical keys, zero keys, needle) and invariants (page-pool permutation,
page size, split count, GQA as repeated-KV MHA, query-token separability,
scratch as extra pages); the e4m3fn decoder is pinned to torch's independent
``float8_e4m3fn`` conversion for all 256 codes. No function is left with
parity unpinned.
"""

from . import e4m3fn  # noqa: F401
from . import kv_write  # noqa: F401
from .paged_decode import (  # noqa: F401
    attend,
    combine_partials,
    kv_head_of,
    logical_kv,
    owns_scratch,
    paged_attention,
    paged_attention_partials,
    split_token_ranges,
    visible_scratch,
)


def run_case(case, num_splits=None):
    """Run the oracle on a ``workloads.DecodeCase`` (host tensors).

    Returns (O, LSE) float64 arrays, or the split partials
    (O_part, LSE_part) when ``num_splits`` is given.
    """
    import numpy as np

    def f64(t):
        return None if t is None else t.to(dtype=__import__("torch").float64).numpy()

    fp8 = case.kv_dtype == "fp8"
    kw = dict(kv_format="fp8" if fp8 else "dense",
              k_scale=None if case.k_scale is None else case.k_scale.numpy(),
              v_scale=None if case.v_scale is None else case.v_scale.numpy(),
              scratch_k=f64(case.scratch_k), scratch_v=f64(case.scratch_v),
              scratch_mask=getattr(case, "scratch_mask", "none"),
              q_lens=None if getattr(case, "q_lens", None) is None else case.q_lens.numpy(),
              scratch_lens=(None if getattr(case, "scratch_lens", None) is None
                            else case.scratch_lens.numpy()),
              kv_layout=getattr(case, "kv_layout", "token"))
    # Dense pools stay float32 (exact for bf16/f16 values, half the memory of
    # float64); rows are widened to float64 as they are gathered.
    kp = case.k_pages.numpy() if fp8 else case.k_pages.float().numpy()
    vp = case.v_pages.numpy() if fp8 else case.v_pages.float().numpy()
    args = (f64(case.q), kp, vp, case.block_table.numpy(),
            case.context_lens.numpy().astype(np.int64), case.scale)
    if num_splits is None:
        return paged_attention(*args, **kw)
    return paged_attention_partials(*args, num_splits, **kw)
