"""MI355X-native jagged attention: GDPA (activation, no row normalisation) and
JFA (online softmax) over variable-length, unpadded batches, forward and
backward, as hand-written gfx950 HIP kernels behind a C ABI."""
