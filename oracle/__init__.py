"""Plain CPU oracle for the hot path of asynchronous block-diffusion drafting.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import, call or execute anything in this package. The product path (the HIP
library and its Python binding) never does, and shares no code with it.

Every function here is the plain definition of what the path computes, written in float64
NumPy from the pages (no blocking, fusion or reordering beyond the definition):

* ``philox``    -- the Philox4x32-10 counter-based generator and the 53-bit uniform built from it
                   (the generator the acceptance test and residual draw consume).
* ``packing``   -- the async draft budget, the order of the packed blocks and the dense
                   visibility mask of one packed draft forward.
* ``attention`` -- softmax attention of the packed queries over their visible keys.
* ``verify``    -- speculative-sampling verification: acceptance ratios, first rejection,
                   residual / bonus sampling, prefix-survival products and the acceptance length.
* ``match``     -- the branch-cache hit test of the verified outcome against the drafted branches.
* ``select``    -- drafter token selection: greedy drafted tokens and the alternative anchors of
                   the branches (the k best tokens of a logit row other than an excluded one).
* ``commit``    -- the accepted slice appended to the paged drafter cache, and the hit branch
                   promoted to the next round's current block.
* ``awl``       -- the acceptance-weighted training loss of the drafter and its gradient.
* ``train_attn`` -- training-time packed attention (response causal, blocks on their anchor's
                   prefix, bidirectional inside a block), forward and backward.

Pages cited in this package:

* [D3D]    the summary page titled "D3D: Decoupled Diffusion Drafting for Asynchronous
           Speculative Decoding" (sections named by their headings: 前置知识 prerequisites,
           核心方法 core method, 方法步骤详情 method steps, ...).
* [DScout] the summary page titled "Factorization-Guided Training and Inference for
           Diffusion-Drafted Speculative Decoding".
* [D3D-abs] the arXiv listing page of D3D (its English abstract).
"""

from . import philox, packing, attention, verify, match, select, commit, awl, train_attn  # noqa: F401
