"""MI355X-native GPU-side decode path of ScoutAttention (block-sparse attention over
block digests, with a GPU/CPU split of the selected blocks).

The compute lives in the HIP library ``libscoutattn.so`` (C ABI, ``include/scoutattn.h``);
``binding`` marshals torch tensors into its calls.  ``workloads`` draws the seeded
synthetic inputs.  The library is loaded on first use and a missing build is an error.
"""
