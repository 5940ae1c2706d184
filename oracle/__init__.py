"""CPU oracle for one denoising step of a bidirectional diffusion LLM under
approximate KV caching.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call, link
or execute this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library (no kernels, headers, helpers, tables or pre/post-processing); the
only thing both sides consume is the seeded input generator's output.

It is deliberately plain and slow: NumPy, one sequence at a time, every
decision-feeding quantity in fp64, each function citing the passage of the
pages it follows.  The pages are four summaries:

* "Polestar - drift-aware cache correction and token commit for efficient
  diffusion LLM inference" (Polestar), sections 1, 2A-2C.
* "Efficient diffusion LLMs via temporal-spatial parallel decoding and
  confidence extrapolation" (TSPD/CE), problem statement and method.
* "Singular proxy for adaptive caching in diffusion language models"
  (SPA-Cache), method steps 1-3.
* The EntropyCache summary, sections 1-2.

Where the pages leave a step open, the reading taken is stated in the
function's docstring.
"""

from .model import *  # noqa: F401,F403
from . import model, decode, brute, budget, polestar, extrapolation  # noqa: F401
