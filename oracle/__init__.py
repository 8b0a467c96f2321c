"""CPU oracle for the quantized DiT-block forward (FastH3 / FastH3 Trim hot path).

TEST INFRASTRUCTURE ONLY. This package is a plain, slow, obviously-correct NumPy statement of what
the hot path computes. It exists to check the HIP path, and only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may import it. The product
path (``quantized_video_diffusion_amd``) never imports, calls or links it, and it imports nothing
from the product path: the two share only the seeded input generators of ``workloads``.

Floating point is float64 unless the method fixes a format (E4M3 codes, INT8 codes, bf16
activations, fp16 AdaLN factors); where a floating-point value decides an integer code the decision
is taken on the fp32 value, as the kernels take it.

Sources (cited by page title and section; no other source defines the method):
  [TRIM]    comfyui-wiki.com news, 2026-10-06, "FastH3 Trim：为 8 GB GPU 打造的剪枝版 8 步 MiniMax H3".
            Sections: "Trim 改变了什么" (what Trim changes: block pruning, timestep conditioning,
            training); "ComfyUI 重打包包含什么" (the repack: formats, calibrated layers);
            "运行速度如何" (speed table and the note under it on the RTX 4090 FP8 path).
  [FARWALK] news.farwalk.ai story on FastVideo FastH3, the authors' thread posts "2/8" ... "8/8";
            post 6/8 is the FP4 calibration statement, post 5/8 the per-network compression.
Format specifications used where the pages only name a format:
  OCP 8-bit Floating Point Specification (OFP8) rev 1.0 — E4M3 ("FN": no infinities, S.1111.111 NaN).
  OCP Microscaling Formats (MX) Specification v1.0 — E2M1 elements, E8M0 shared scales, the
  shared-exponent rule floor(log2(amax)) - emax_elem.

Where the pages leave a step open, the reading taken is stated in the docstring of the function
that takes it. Every function here is pinned by a CPU test under tests/ against a closed form, a
brute force, a special case or an invariant.
"""

from . import codecs, quant, adaln, gemm, attention, block, sampler  # noqa: F401
