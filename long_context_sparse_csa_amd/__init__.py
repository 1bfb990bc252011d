"""MI355X-native DeepSeek-V4 hybrid compressed attention (CSA + HCA).

The compute runs in hand-written HIP kernels for gfx950 inside the C-ABI
library `libv4attn.so` (declared in include/v4attn.h).  `ops` is the thin
Python binding over it (argument marshalling only; it loads the library on
first use and raises if it is missing).  `configs` names the workloads and
`synth` draws their seeded inputs.
"""

import os

PACKAGE_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PACKAGE_DIR, "libv4attn.so")

