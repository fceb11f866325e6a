// Definitions shared by the attention kernels (attention_fwd.hip, attention_frag.hip).
#pragma once
#include "internal.hpp"

namespace pisa {

enum { MODE_DROP = 0, MODE_PISA = 1, MODE_PWT = 2, MODE_LITERAL = 3, MODE_PWT_ROW = 4 };

// Lazy rescaling threshold of the online softmax, in log2 units: the running max only
// moves when a logit exceeds it by more than kTau, so exponentials stay <= 2^kTau and
// the accumulators are rescaled on few tiles. All state is scaled by 2^-m.
constexpr float kTau = 8.f;

// Row permutation that makes MFMA accumulators reusable as the next product's B operand:
// the lane with A-row R of a 32-row m-tile loads row feed_row(R); accumulator register r
// of m-tile mt in lane half g then holds row acc_key(mt, r, g), and registers
// [KH*ks, KH*ks + KH) hold rows KI*ks + KH*g + [0, KH), the B operand of k-step ks.
template <class M>
__device__ __forceinline__ int feed_row(int R) {
  const int r = 4 * (R >> 3) + (R & 3), gg = (R >> 2) & 1;
  return M::KI * (r / M::KH) + M::KH * gg + (r % M::KH);
}
template <class M>
__device__ __forceinline__ int acc_key(int mt, int r, int g) {
  return 32 * mt + M::KI * (r / M::KH) + M::KH * g + (r % M::KH);
}

// bf16 DROP / PISA / PWT: register-streamed kernel over operand-order tiles.
hipError_t launch_attention_frag(int mode, const AttnArgs& a, hipStream_t s);
// bf16 PWT_ROW: virtual tokens with the per-row w, merged into O / lse of a DROP pass.
hipError_t launch_virtual_row(const AttnArgs& a, hipStream_t s);

}  // namespace pisa
