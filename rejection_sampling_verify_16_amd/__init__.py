"""MI355X-native speculative-decoding verify sampler (libspecverify) and its inputs."""
