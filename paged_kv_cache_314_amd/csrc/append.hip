// KV-cache append: write the new tokens' K/V rows into their cache blocks.
//
// Token t of sequence b lives in block blockTables[b][t / blockSize], slot
// t % blockSize (aclnnFusedInferAttentionScoreV3, Constraints, paged attention scenario);
// the seqLen[b] new tokens are the sequence's last positions (PrefixEncoder, Members:
// kvSeqLen counts the cached prefix plus the new tokens).  One workgroup copies up to
// kAppendRows tokens of one sequence: every (token, kv head) row of headSize elements as
// 16-byte chunks, consecutive lanes on consecutive chunks of a row, for K and V.  A pure
// copy: the bytes of the cache equal the bytes of the new rows.
#include "pa_device.h"
#include "pa_internal.h"
#include "pa_kernels.h"

namespace pa {

namespace {

__global__ void __launch_bounds__(256) append_kernel(AppendArgs a) {
    const AppendItem it = a.items[blockIdx.x];
    const int ch = a.row_chunks;                  // 16-byte chunks per (token, kv head) row
    const int per_tok = a.kv_heads * ch;
    const int total = it.count * per_tok;
    const int32_t* trow = a.table + static_cast<int64_t>(it.b) * a.table_stride;
    for (int e = threadIdx.x; e < total; e += blockDim.x) {
        const int r = e / per_tok;
        const int rem = e - r * per_tok;
        const int h = rem / ch;
        const int c = rem - h * ch;
        const int pos = it.pos0 + r;
        const int blk = trow[pos / a.block_size];
        const int slot = pos - (pos / a.block_size) * a.block_size;
        const int64_t row = it.row0 + r;
        const int64_t kdst = static_cast<int64_t>(blk) * a.k_blk_stride + static_cast<int64_t>(slot) * a.k_slot_stride +
                             static_cast<int64_t>(h) * a.k_head_stride;
        const int64_t vdst = static_cast<int64_t>(blk) * a.v_blk_stride + static_cast<int64_t>(slot) * a.v_slot_stride +
                             static_cast<int64_t>(h) * a.v_head_stride;
        const int64_t ksrc = row * a.knew_tok_stride + static_cast<int64_t>(h) * a.knew_head_stride;
        const int64_t vsrc = row * a.vnew_tok_stride + static_cast<int64_t>(h) * a.vnew_head_stride;
        // strides are in elements; every offset is a multiple of 16 bytes
        const char* kn = static_cast<const char*>(a.knew) + ksrc * a.elem_bytes + 16 * c;
        const char* vn = static_cast<const char*>(a.vnew) + vsrc * a.elem_bytes + 16 * c;
        char* kc = static_cast<char*>(a.kcache) + kdst * a.elem_bytes + 16 * c;
        char* vc = static_cast<char*>(a.vcache) + vdst * a.elem_bytes + 16 * c;
        const u32x4 kx = *reinterpret_cast<const u32x4*>(kn);
        const u32x4 vx = *reinterpret_cast<const u32x4*>(vn);
        *reinterpret_cast<u32x4*>(kc) = kx;
        *reinterpret_cast<u32x4*>(vc) = vx;
    }
}

}  // namespace

hipError_t launch_append(const AppendArgs& a, int n_items, hipStream_t stream, hipEvent_t t0,
                         hipEvent_t t1) {
    if (n_items <= 0) return hipSuccess;
    launch_256(append_kernel, n_items, stream, t0, t1, a);
    return hipGetLastError();
}

}  // namespace pa
