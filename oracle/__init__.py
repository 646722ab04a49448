"""CPU oracle for the VDN-H3 hybrid attention layer.

THIS PACKAGE IS TEST INFRASTRUCTURE.  Only the tests, the package's smoke check and the
bench's CPU-baseline leg may import it.  The product path (the HIP library and its
Python binding) never imports, calls or links anything here, and nothing here imports
the product package: the two share no code.

What it computes follows the VDN-MiniMax-H3 article on modelscope.csdn.net ("VDN-MiniMax-H3
开源：全新混合注意力加速视频生成"), sections "局部精确计算，远程线性记忆" (local exact
softmax, long-range linear memory) and "独立门控，融合两条注意力分支" (per-branch gates and
output projections).  Plain numpy, float64 throughout; a library matmul is the only
primitive used as a step.

Readings taken where the article is silent or ambiguous (each is also the HIP path's):

* Chunks start at frame 0 (chunk of frame f is f // C); the last chunk may be short.
* The window of a chunk is the chunk and R = 1 chunk on each side, clipped at the clip
  edges (no wrap-around, no shifted window).
* The first and last frames are anchors.  Anchor query frames read every frame by
  softmax, and their forward and backward linear states hold text only.
* Key sets are set unions: an anchor inside the window is counted once.
* Every text token is a key of every query (no padding); text and audio tokens are not
  queries of this layer.
* Linear attention: feature map identity, additive state, no normaliser, no scale; the
  state of a frame is the sum over its tokens of k^T v, updated once per frame.
* Forward state = text/2 + sum of the frames before the window (anchors excluded);
  backward state = text/2 + sum of the frames after it (anchors excluded); the two reads
  q.S_fwd and q.S_bwd are added.
* Softmax scale d**-0.5.  Gates are elementwise sigmoids of given logits, applied to
  each head's output before its projection.  RMSNorm runs over head_dim per (token,
  head) with a per-(head, channel) weight and eps = 1e-6.  Projections have no bias and
  add into the residual stream as a plain sum.

Parity pins: every function here is pinned by a CPU test (tests/test_oracle_*.py) to
something other than itself — the article's frame-7 example, hand-derived set tables,
library attention and RMSNorm routines, brute-force loops and closed-form invariants.
"""
from . import layer, mxfp8, sets  # noqa: F401
