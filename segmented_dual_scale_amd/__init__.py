"""segmented_dual_scale_amd: the DualScale x SegLinear W8A8 linear layer on
MI355X (gfx950).  The Python binding over the C-ABI library is added with
the library itself; ``workloads`` holds the seeded input generators."""
