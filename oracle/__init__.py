"""FP64 CPU oracle for the MXFP4 latent-MoE routed-expert forward. Test infrastructure only."""
