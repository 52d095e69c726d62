// Fused disentangled-attention forward: the 16-bit instances at head dim 128.
//
// The forward's kernels are one template (dattn_fwd.hip). This unit
// instantiates only the fp16/bf16 d = 128 ones, so that the build can
// schedule them with the default machine scheduler while the rest of the
// forward uses the max-ilp scheduler: measured on MI355X, max-ilp is faster
// for every other instance (strict fp32 d = 128 by 8%, the long bf16 d = 64
// shapes by 1-2%) and 2% slower for these.
#define DATTN_FWD_H16_D128_UNIT 1
#include "dattn_fwd.hip"
