"""MI355X-native CSA / HCA hybrid-attention hot path.

`binding` wraps the C ABI of libcsa.so (include/csa.h); `synth` draws the
seeded synthetic workloads; `path` chains the entry points into whole CSA /
HCA prefill and decode steps.  Importing the package does not load the
library; the first call through `binding` does, and fails loudly if the
library has not been built.
"""
