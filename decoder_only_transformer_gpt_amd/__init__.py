"""MI355X (gfx950) library for one nanochat GPT pretraining step, forward and
backward. The C ABI is in include/gpt.h; ``_lib`` binds it, ``model.GPT`` wraps
it with torch-owned device memory, ``workloads`` names the configurations."""
