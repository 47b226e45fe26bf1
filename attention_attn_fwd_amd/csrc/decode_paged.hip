// The paged-cache instantiations of the split-KV decode kernel (block-table
// and ring-buffer caches), compiled apart from the packed-cache kernel so
// that the build can schedule each with its own instruction scheduler; the
// kernel source is the one in decode.hip.
#define GPTOSS_DECODE_PAGED_UNIT 1
#include "decode.hip"
