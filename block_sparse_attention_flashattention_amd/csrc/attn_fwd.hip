// Forward-kernel dispatch by query-tile height. All kernels run the same
// per-wave arithmetic (wave_engine.h). Three use eight waves whose two groups
// alternate between MFMA and softmax phases and differ in how the 256 row
// slots of the eight waves are filled:
//   256-row tiles: one KV stream shared by all waves    (attn_fwd_pp.hip)
//   128-row tiles: two KV streams, merged at the end     (attn_fwd_2s.hip;
//                  over 128-key tiles, whole-tile streams: attn_fwd_2t.hip)
//    64-row tiles: four KV streams, merged at the end    (attn_fwd_4s.hip)
// With many 64- or 128-row work items, the independent-wave kernel
// (attn_fwd_iw.hip: one stream, several workgroups per compute unit) runs
// instead.
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
    // Many work items: independent waves, several workgroups per compute unit.
    // Few: all eight waves of a workgroup on one tile, over two or four streams.
    if (p.splits > 1 || (int64_t)p.n_work >= (int64_t)kIwItemsPerCu * device_cu_count())
        return launch_fwd_iw(block_q, head_dim, p, stream);
    if (block_q == 128) return block_kv == 128 ? launch_fwd_2t(head_dim, p, stream) : launch_fwd_2s(block_kv, head_dim, p, stream);
    return launch_fwd_4s(block_kv, head_dim, p, stream);
}

}  // namespace vsa
