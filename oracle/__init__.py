"""CPU oracle for VideoMLA latent-KV chunk attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, links or runs
anything from this package; only the tests, the smoke entry point and the
CPU-baseline leg of the benchmark do.  It shares no code with the HIP path:
it receives plain arrays and geometry numbers and returns arrays.

Source: "VideoMLA: Low-Rank Latent KV Cache for Minute-Scale Autoregressive
Video Diffusion" (paper text, sections 3-4 and appendices C.1, D.1, D.4, D.5).
The equations that define the latent c_t^KV, the per-head reconstruction and
the decoupled key k_t^R are referenced but absent from the available text; the
oracle follows the Multi-Head Latent Attention form the paper builds on
(DeepSeek-V2, reference [14] of the paper).  Each reading of a silent or
garbled point is stated where it is used.

Modules
  mla    -- numpy float64 implementation (explicit up-projection, naive softmax)
  brute  -- pure-Python loop implementation for tiny inputs
  ring   -- sliding-window frame bookkeeping (integer, exact)
  sizes  -- cache-size arithmetic of the paper's per-token layout
"""
from . import brute, mla, ring, sizes  # noqa: F401
