// Multi-token queries: speculative verification (the k guessed tokens a target
// model checks in one pass, "Scaling inference with vLLM", speculative decoding
// paragraph) and prefill chunks ("Local_LLM_03_vLLM_Architecture",
// chunked-prefill slide).  The n query rows of a sequence are its last n
// positions; with the causal mask row i sees keys t <= L - n + i.
#include "pa_common.h"

namespace pa {

// Vector-ALU path: every query row runs the decode kernel over its own visible
// length (per-row mode of launch_decode).
hipError_t launch_multiq(int dtype, int head_dim, int block_size, int group, int num_seqs,
                         const AttnArgs& a, hipStream_t st, const KernelEvents& ev) {
  return launch_decode(dtype, head_dim, block_size, group, num_seqs, a, st, ev);
}

}  // namespace pa
