"""CPU oracle of the denoising step (test infrastructure only; see dgd_oracle)."""
