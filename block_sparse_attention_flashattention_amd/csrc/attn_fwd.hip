// Forward-kernel dispatch by query-tile height. All three kernels run the
// same per-wave arithmetic (wave_engine.h) with eight waves whose two groups
// alternate between MFMA and softmax phases; they differ in how the 256 row
// slots of the eight waves are filled:
//   256-row tiles: one KV stream shared by all waves    (attn_fwd_pp.hip)
//   128-row tiles: two KV streams, merged at the end     (attn_fwd_2s.hip)
//    64-row tiles: four KV streams, merged at the end    (attn_fwd_4s.hip)
#include "vsa_internal.h"

namespace vsa {

bool fwd_supported(int block_q, int block_kv, int head_dim) {
    const bool bq = block_q == 64 || block_q == 128 || block_q == 256;
    const bool bkv = block_kv == 64 || block_kv == 128;
    const bool d = head_dim == 64 || head_dim == 128;
    return bq && bkv && d;
}

hipError_t launch_fwd(int block_q, int block_kv, int head_dim, const FwdParams& p, hipStream_t stream) {
    if (!fwd_supported(block_q, block_kv, head_dim)) return hipErrorInvalidValue;
    if (block_q == 256) return launch_fwd_pp(block_kv, head_dim, p, stream);
    if (block_q == 128) return launch_fwd_2s(block_kv, head_dim, p, stream);
    return launch_fwd_4s(block_kv, head_dim, p, stream);
}

}  // namespace vsa
