"""Seeded synthetic inputs shared by the oracle tests, the GPU tests and the
bench: workload shapes (``configs``), expert weight blobs (``experts``) and
activations / router-logit traces (``traces``).  Input generation only; none of
the MoE layer's arithmetic lives here."""
