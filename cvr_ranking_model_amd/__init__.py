"""MI355X-native candidate scoring: mean-pooled embedding gather + DLRM-style MLP or HyFormer-style CVR stack.

Importing the package loads nothing native; :mod:`cvr_ranking_model_amd.cvr` loads the HIP library.
"""
__all__ = ["synth", "cvr"]
