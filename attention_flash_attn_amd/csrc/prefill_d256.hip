// Prefill kernels at head dim 256, compiled in a translation unit of their own so
// that they can take another machine-scheduler strategy than the other head dims
// (the build passes it for this file); the kernel source is the same.
#define ATTN_PREFILL_D256_UNIT 1
#include "prefill.hip"
