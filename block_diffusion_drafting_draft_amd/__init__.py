"""MI355X-native hot path of asynchronous block-diffusion speculative decoding."""
