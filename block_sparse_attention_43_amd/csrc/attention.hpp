// Definitions shared by the attention kernels (attention_fwd.hip, attention_frag.hip).
#pragma once
#include "internal.hpp"

namespace pisa {

enum { MODE_DROP = 0, MODE_PISA = 1, MODE_PWT = 2, MODE_LITERAL = 3, MODE_PWT_ROW = 4 };

// Lazy rescaling threshold of the online softmax, in log2 units: the running max only
// moves when a logit exceeds it by more than kTau, so exponentials stay <= 2^kTau and
// the accumulators are rescaled on few tiles. All state is scaled by 2^-m.
constexpr float kTau = 8.f;

// bf16 DROP / PISA / PWT: register-streamed kernel over operand-order tiles.
hipError_t launch_attention_frag(int mode, const AttnArgs& a, hipStream_t s);

}  // namespace pisa
