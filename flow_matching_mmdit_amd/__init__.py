"""MI355X-native AuraFlow transformer forward (hand-written HIP kernels behind a C ABI).

``flow_matching_mmdit_amd.binding`` loads lib/libauraflow.so and exposes the
C-ABI calls of include/auraflow.h plus the ``AuraFlowModel`` tensor wrapper.
Build the library with ``python -m flow_matching_mmdit_amd.build``.
"""
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "lib", "libauraflow.so")
HEADER_PATH = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "auraflow.h")
