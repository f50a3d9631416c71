"""ttsbb: forward pass of a Qwen3-0.6B-shaped TTS backbone as hand-written HIP kernels for
AMD MI355X (gfx950), behind the C ABI of include/ttsbb.h.  ``codec_token_tts_amd.ttsbb``
is the Python binding; ``codec_token_tts_amd.build`` compiles the library."""
