// Block copies and the accept walk of speculative verify rounds.
//
// TensorFold page, section on the GPU accept kernel: a verify round closes on
// the device. Each draft token is compared with the target's choice, the
// accepted path follows from the root the first child whose draft equals the
// choice, and a rollback restores the KV cache after that path. The host pool
// (kv_pool_truncate) does the block bookkeeping of a rollback; kv_copy_blocks
// copies a shared block that a truncated sequence must stop sharing;
// kv_accept_paths walks every sequence's window at once.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "pagedkv.h"
#include "status.h"

namespace pkv {
namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// One workgroup per (src, dst) pair; a block of one pool is `pieces`
// 16-byte pieces (every KV head's tile), copied in order by 256 lanes.
__global__ __launch_bounds__(256) void copy_blocks_kernel(uint8_t *kp, uint8_t *vp, const int32_t *src,
                                                          const int32_t *dst, int num_blocks, int64_t pieces) {
    const int i = blockIdx.x;
    const int a = src[i], b = dst[i];
    if (a < 0 || a >= num_blocks || b < 0 || b >= num_blocks) return;
    const int64_t bytes = pieces * 16;
    const u32x4_t *ks = reinterpret_cast<const u32x4_t *>(kp + a * bytes);
    const u32x4_t *vs = reinterpret_cast<const u32x4_t *>(vp + a * bytes);
    u32x4_t *kd = reinterpret_cast<u32x4_t *>(kp + b * bytes);
    u32x4_t *vd = reinterpret_cast<u32x4_t *>(vp + b * bytes);
    for (int64_t p = threadIdx.x; p < pieces; p += 256) {
        kd[p] = ks[p];
        vd[p] = vs[p];
    }
}

// One lane per sequence. The walk makes at most q_len moves, so it ends
// whatever the parents hold.
__global__ __launch_bounds__(64) void accept_kernel(const int32_t *parents, const int32_t *drafts,
                                                   const int32_t *choices, const int32_t *root_choices,
                                                   const int32_t *qsl, int num_seqs, int32_t *path, int32_t *path_len,
                                                   int32_t *bonus) {
    const int s = blockIdx.x * 64 + threadIdx.x;
    if (s >= num_seqs) return;
    const int q0 = qsl[s];
    const int W = max(qsl[s + 1] - q0, 0);
    for (int r = 0; r < W; ++r) path[q0 + r] = -1;
    int cur = -1, want = root_choices[s], len = 0;
    for (int step = 0; step < W; ++step) {
        int nxt = -1;
        for (int r = 0; r < W; ++r)
            if (parents[q0 + r] == cur && drafts[q0 + r] == want) {
                nxt = r;
                break;
            }
        if (nxt < 0) break;
        path[q0 + len] = nxt;
        ++len;
        cur = nxt;
        want = choices[q0 + nxt];
    }
    path_len[s] = len;
    bonus[s] = want;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace
}  // namespace pkv

extern "C" {

int kv_copy_blocks(void *k_pool, void *v_pool, const int32_t *src, const int32_t *dst, int32_t n,
                   int32_t num_blocks, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                   int32_t dtype, void *hip_stream) {
    using namespace pkv;
    if (block_size != 16) PKV_FAIL(KV_EUNSUPPORTED, "kv_copy_blocks: block_size %d not supported (16)", block_size);
    if (n < 0 || num_blocks < 0 || num_kv_heads <= 0 || head_dim <= 0 || head_dim % 16 || head_dim > 256)
        PKV_FAIL(KV_EINVAL, "kv_copy_blocks: invalid size");
    int64_t tile;
    if (dtype == KV_BF16) tile = 16LL * head_dim * 2;
    else if (dtype == KV_F32) tile = 16LL * head_dim * 4;
    else if (dtype == KV_FP8) tile = 16LL * head_dim + 64;
    else if (dtype == KV_FP4) tile = 8LL * head_dim + 64;
    else PKV_FAIL(KV_EUNSUPPORTED, "kv_copy_blocks: dtype %d not supported", dtype);
    if (n == 0) return KV_OK;
    if (!k_pool || !v_pool || !src || !dst) PKV_FAIL(KV_EINVAL, "kv_copy_blocks: required pointer is NULL");
    if (!aligned16(k_pool) || !aligned16(v_pool)) PKV_FAIL(KV_EINVAL, "kv_copy_blocks: pools must be 16-byte aligned");
    const int64_t pieces = tile * num_kv_heads / 16;
    hipStream_t st = reinterpret_cast<hipStream_t>(hip_stream);
    (void)hipGetLastError();
    hipLaunchKernelGGL(copy_blocks_kernel, dim3((unsigned)n), dim3(256), 0, st, static_cast<uint8_t *>(k_pool),
                       static_cast<uint8_t *>(v_pool), src, dst, num_blocks, pieces);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) PKV_FAIL(KV_EDEVICE, "kv_copy_blocks: launch failed: %s", hipGetErrorString(e));
    return KV_OK;
}

int kv_accept_paths(const int32_t *parents, const int32_t *draft_tokens, const int32_t *choices,
                    const int32_t *root_choices, const int32_t *query_start_loc, int32_t num_seqs,
                    int32_t *path, int32_t *path_len, int32_t *bonus, void *hip_stream) {
    using namespace pkv;
    if (num_seqs < 0) PKV_FAIL(KV_EINVAL, "kv_accept_paths: num_seqs %d < 0", num_seqs);
    if (num_seqs == 0) return KV_OK;
    if (!parents || !draft_tokens || !choices || !root_choices || !query_start_loc || !path || !path_len || !bonus)
        PKV_FAIL(KV_EINVAL, "kv_accept_paths: required pointer is NULL");
    hipStream_t st = reinterpret_cast<hipStream_t>(hip_stream);
    (void)hipGetLastError();
    hipLaunchKernelGGL(accept_kernel, dim3((unsigned)((num_seqs + 63) / 64)), dim3(64), 0, st, parents, draft_tokens,
                       choices, root_choices, query_start_loc, num_seqs, path, path_len, bonus);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) PKV_FAIL(KV_EDEVICE, "kv_accept_paths: launch failed: %s", hipGetErrorString(e));
    return KV_OK;
}

}  // extern "C"
