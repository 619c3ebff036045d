"""Group-shared importance-sampled permuted block-sparse attention (InstaGen) on MI355X.

The compute path is the HIP library libisg.so (C ABI in include/isg.h); the
binding in ``isg`` only marshals torch device tensors into it.  Importing the
package does not load the library; the first ``isg`` call does.
"""
__all__ = ["isg", "synth", "workloads"]
