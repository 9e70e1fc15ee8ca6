// QK-norm + NeoX RoPE + paged scatter-write in one pass.
//
// TensorSharp "高级功能" page: for Qwen 3.5/3.6 one kernel applies QK-Norm
// and NeoX RoPE on the prefill path, and the batched forward pairs the
// projection with the paged K/V scatter-write. Here the three are one launch:
// every (token, head) row of Q and K is RMS-normalized over the head
// dimension with per-dimension weights (offset + w), its first rotary_dim
// dimensions are turned in NeoX pairs (i, i + rotary_dim / 2) by the angle
// pos * theta^(-2i / rotary_dim), and the result is rounded once to bf16; Q
// goes to q_out, K and V (unchanged) into the bf16 pools at their slots.
//
// Workgroup: 16 consecutive tokens x up to kHeadsPerWG rows of the Q, K and
// V heads (in that order). Lane group t (16 lanes) owns token t; lane p of it
// owns the D/16 consecutive dimensions p*D/16 .. p*D/16 + D/16 - 1, so that a
// row loads and stores in 16-byte pieces and the K tile layout
// [D/8][16][8] takes whole pieces. The NeoX partner of a dimension sits
// rotary_dim/2 / (D/16) lanes away, in the same register. The angles are
// computed once per workgroup: the angle in float64, reduced to [-pi, pi],
// then sine and cosine in float32.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "pagedkv.h"
#include "status.h"

namespace pkv {
namespace {

constexpr int kBlk = 16;
constexpr int kHeadsPerWG = 4;

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

struct ProdArgs {
    const uint16_t *q, *k, *v;  // [n][H][D] bf16
    const int32_t *pos;         // [n]
    const uint16_t *qw, *kw;    // [D] bf16 or null
    const int32_t *slots;       // [n]
    uint16_t *q_out;            // [n][Hq][D]
    uint16_t *kp, *vp;          // pools
    int n, Hq, Hkv, num_blocks, rotary_dim;
    float eps, weight_offset;
    double log2_theta;
};

__device__ inline float bf16_to_f32(uint16_t b) { return __builtin_bit_cast(float, (uint32_t)b << 16); }

// Nearest bf16, ties to even (finite inputs).
__device__ inline uint16_t f32_to_bf16(float f) {
    const uint32_t u = __builtin_bit_cast(uint32_t, f);
    return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

template <int CPT>
__device__ inline void load_row(const uint16_t *src, uint16_t (&x)[CPT]) {
    if constexpr (CPT == 4) {
        const u32x2_t w = *reinterpret_cast<const u32x2_t *>(src);
        __builtin_memcpy(x, &w, 8);
    } else {
#pragma unroll
        for (int c = 0; c < CPT; c += 8) {
            const u32x4_t w = *reinterpret_cast<const u32x4_t *>(src + c);
            __builtin_memcpy(x + c, &w, 16);
        }
    }
}

template <int CPT>
__device__ inline void store_row(uint16_t *dst, const uint16_t (&x)[CPT]) {
    if constexpr (CPT == 4) {
        u32x2_t w;
        __builtin_memcpy(&w, x, 8);
        *reinterpret_cast<u32x2_t *>(dst) = w;
    } else {
#pragma unroll
        for (int c = 0; c < CPT; c += 8) {
            u32x4_t w;
            __builtin_memcpy(&w, x + c, 16);
            *reinterpret_cast<u32x4_t *>(dst + c) = w;
        }
    }
}

template <int D>
__global__ __launch_bounds__(256) void qknorm_rope_scatter_kernel(ProdArgs A) {
    constexpr int CPT = D / 16;
    const int tid = threadIdx.x;
    const int t = tid >> 4, part = tid & 15, lane = tid & 63;
    const int i0 = blockIdx.x * kBlk;
    const int tok = i0 + t;
    const bool have = tok < A.n;
    const int half = A.rotary_dim / 2;
    const int shift = half / CPT;  // lanes between NeoX partners

    __shared__ int s_slot[kBlk];
    __shared__ int s_full;
    __shared__ __attribute__((aligned(16))) uint16_t sv[kBlk][D];
    __shared__ double s_inv_freq[D / 2];  // theta^(-2i / rotary_dim), i < rotary_dim / 2
    if (tid < half) s_inv_freq[tid] = exp2(-(2.0 * tid / A.rotary_dim) * A.log2_theta);
    if (tid < kBlk) {
        const int i = i0 + tid;
        const int sl = i < A.n ? A.slots[i] : -1;
        s_slot[tid] = (sl >= 0 && sl < A.num_blocks * kBlk) ? sl : -1;
    }

    // The rows of the workgroup's heads are loaded first, so that their
    // latency overlaps the angle arithmetic.
    const int Htot = A.Hq + 2 * A.Hkv;
    const int h0 = blockIdx.y * kHeadsPerWG;
    const int nh = min(Htot - h0, kHeadsPerWG);
    auto kind_of = [&](int hh) { return hh < A.Hq ? 0 : hh < A.Hq + A.Hkv ? 1 : 2; };  // Q, K, V
    auto head_of = [&](int hh) { return hh < A.Hq ? hh : hh < A.Hq + A.Hkv ? hh - A.Hq : hh - A.Hq - A.Hkv; };
    uint16_t xs[kHeadsPerWG][CPT];
#pragma unroll
    for (int j = 0; j < kHeadsPerWG; ++j) {
        const int hh = h0 + min(j, nh - 1);
        const int kind = kind_of(hh), head = head_of(hh);
        const int H = kind == 0 ? A.Hq : A.Hkv;
        const uint16_t *src = (kind == 0 ? A.q : kind == 1 ? A.k : A.v) +
                              ((size_t)(have ? tok : 0) * H + head) * D + part * CPT;
        load_row<CPT>(src, xs[j]);
    }

    __syncthreads();
    // cosine and sine of the lane's dimensions (identity past rotary_dim):
    // lanes of the lower half of each pair compute them, their partners
    // `shift` lanes up take them by shuffle
    float cs[CPT], sn[CPT];
    {
        const double p = have ? (double)A.pos[tok] : 0.0;
        const bool lower = part * CPT < half;
#pragma unroll
        for (int e = 0; e < CPT; ++e) {
            const int c = part * CPT + e;
            float cv = 1.f, sv_ = 0.f;
            if (lower) {
                const double ang = p * s_inv_freq[c];
                const double turns = rint(ang * (1.0 / (2.0 * M_PI)));
                sincosf((float)fma(-turns, 2.0 * M_PI, ang), &sv_, &cv);
            }
            const int src = lower || !shift ? lane : lane - shift;
            const float co = __shfl(cv, src, 64), so = __shfl(sv_, src, 64);
            const bool rot = c < A.rotary_dim;
            cs[e] = rot ? co : 1.f;
            sn[e] = rot ? so : 0.f;
        }
    }
    if (tid < 64) {
        const int sl0 = s_slot[0];
        const bool ok = tid >= kBlk || (s_slot[tid] >= 0 && s_slot[tid] == sl0 + tid && sl0 % kBlk == 0);
        const bool full = __all(ok);
        if (tid == 0) s_full = full;
    }
    __syncthreads();
    const int slot = s_slot[t];

#pragma unroll
    for (int j = 0; j < kHeadsPerWG; ++j) {
        if (j >= nh) break;  // uniform over the workgroup
        const int hh = h0 + j;
        const int kind = kind_of(hh), head = head_of(hh);
        uint16_t(&x)[CPT] = xs[j];
        if (kind != 2) {
            float y[CPT];
            float ss = 0.f;
#pragma unroll
            for (int e = 0; e < CPT; ++e) {
                y[e] = bf16_to_f32(x[e]);
                ss = fmaf(y[e], y[e], ss);
            }
#pragma unroll
            for (int o = 8; o >= 1; o >>= 1) ss += __shfl_xor(ss, o, 64);
            const float inv = 1.f / __fsqrt_rn(__fdiv_rn(ss, (float)D) + A.eps);
            const uint16_t *wt = kind == 0 ? A.qw : A.kw;
#pragma unroll
            for (int e = 0; e < CPT; ++e) {
                const float w = wt ? A.weight_offset + bf16_to_f32(wt[part * CPT + e]) : 1.f;
                y[e] = (y[e] * inv) * w;
            }
            // NeoX pairs: the lower half takes its partner from `shift` lanes up,
            // the upper half from `shift` lanes down (same register)
            const bool lower = part * CPT < half;
            const int src_lane = lower ? lane + shift : lane - shift;
#pragma unroll
            for (int e = 0; e < CPT; ++e) {
                const float other = __shfl(y[e], shift ? src_lane : lane, 64);
                const float rot = lower ? y[e] * cs[e] - other * sn[e] : y[e] * cs[e] + other * sn[e];
                x[e] = f32_to_bf16(part * CPT + e < A.rotary_dim ? rot : y[e]);
            }
        }
        if (kind == 0) {
            if (have) store_row<CPT>(A.q_out + ((size_t)tok * A.Hq + head) * D + part * CPT, x);
            continue;
        }
        if (kind == 1) {
            // K tile [D/8][16][8]: the lane's dimensions are whole 8-element pieces
            if (have && slot >= 0) {
                uint16_t *tile = A.kp + ((size_t)(slot / kBlk) * A.Hkv + head) * kBlk * D;
                const int o = slot % kBlk;
#pragma unroll
                for (int c = 0; c < CPT; c += 8 < CPT ? 8 : CPT) {
                    const int c0 = part * CPT + c;
                    uint16_t *dst = tile + ((c0 / 8) * kBlk + o) * 8 + c0 % 8;
                    if constexpr (CPT == 4) {
                        u32x2_t w;
                        __builtin_memcpy(&w, x + c, 8);
                        *reinterpret_cast<u32x2_t *>(dst) = w;
                    } else {
                        u32x4_t w;
                        __builtin_memcpy(&w, x + c, 16);
                        *reinterpret_cast<u32x4_t *>(dst) = w;
                    }
                }
            }
            continue;
        }
        // V tile [D][16]
        if (s_full) {
            store_row<CPT>(&sv[t][part * CPT], x);
            __syncthreads();
            uint16_t *tile = A.vp + ((size_t)(s_slot[0] / kBlk) * A.Hkv + head) * kBlk * D;
            for (int pc = tid; pc < 2 * D; pc += 256) {  // piece pc: channel pc/2, tokens 8 (pc&1) .. +7
                const int c = pc >> 1, t0 = (pc & 1) * 8;
                uint16_t b[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) b[e] = sv[t0 + e][c];
                u32x4_t w;
                __builtin_memcpy(&w, b, 16);
                *reinterpret_cast<u32x4_t *>(tile + (size_t)pc * 8) = w;
            }
            __syncthreads();
        } else if (have && slot >= 0) {
            uint16_t *tile = A.vp + ((size_t)(slot / kBlk) * A.Hkv + head) * kBlk * D;
#pragma unroll
            for (int e = 0; e < CPT; ++e) tile[(size_t)(part * CPT + e) * kBlk + slot % kBlk] = x[e];
        }
    }
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace
}  // namespace pkv

extern "C" {

int kv_qknorm_rope_scatter(const void *q, const void *k, const void *v, const int32_t *positions,
                           const void *q_norm_weight, const void *k_norm_weight, float eps, float weight_offset,
                           float rope_theta, int32_t rotary_dim, const int32_t *slot_mapping, int32_t n,
                           void *q_out, void *k_pool, void *v_pool, int32_t num_blocks, int32_t num_q_heads,
                           int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t dtype,
                           void *hip_stream) {
    using namespace pkv;
    if (dtype != KV_BF16) PKV_FAIL(KV_EUNSUPPORTED, "kv_qknorm_rope_scatter: dtype %d not supported (bf16)", dtype);
    if (block_size != kBlk)
        PKV_FAIL(KV_EUNSUPPORTED, "kv_qknorm_rope_scatter: block_size %d not supported (16)", block_size);
    if (head_dim != 64 && head_dim != 128 && head_dim != 256)
        PKV_FAIL(KV_EUNSUPPORTED, "kv_qknorm_rope_scatter: head_dim %d not supported (64, 128, 256)", head_dim);
    if (n < 0 || num_blocks < 0 || num_q_heads <= 0 || num_kv_heads <= 0)
        PKV_FAIL(KV_EINVAL, "kv_qknorm_rope_scatter: invalid size");
    if (rotary_dim < 0 || rotary_dim > head_dim || rotary_dim % 2 || (rotary_dim / 2) % (head_dim / 16))
        PKV_FAIL(KV_EINVAL,
                 "kv_qknorm_rope_scatter: rotary_dim %d must be even, at most head_dim and rotary_dim/2 a multiple "
                 "of head_dim/16",
                 rotary_dim);
    if (!(rope_theta > 0.f) || !std::isfinite(rope_theta) || !(eps >= 0.f) || !std::isfinite(eps) ||
        !std::isfinite(weight_offset))
        PKV_FAIL(KV_EINVAL, "kv_qknorm_rope_scatter: rope_theta must be positive, eps >= 0, all finite");
    if (n == 0) return KV_OK;
    if (!q || !k || !v || !positions || !slot_mapping || !q_out || !k_pool || !v_pool)
        PKV_FAIL(KV_EINVAL, "kv_qknorm_rope_scatter: required pointer is NULL");
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(q_out) || !aligned16(k_pool) ||
        !aligned16(v_pool))
        PKV_FAIL(KV_EINVAL, "kv_qknorm_rope_scatter: rows, q_out and pools must be 16-byte aligned");
    if ((int64_t)num_blocks * kBlk > INT32_MAX) PKV_FAIL(KV_EINVAL, "kv_qknorm_rope_scatter: pool too large");
    const int64_t groups = ((int64_t)n + kBlk - 1) / kBlk;
    const int64_t hgroups = ((int64_t)num_q_heads + 2 * num_kv_heads + kHeadsPerWG - 1) / kHeadsPerWG;
    if (groups > INT32_MAX || hgroups > 65535) PKV_FAIL(KV_EINVAL, "kv_qknorm_rope_scatter: too many tokens or heads");
    ProdArgs A;
    A.q = static_cast<const uint16_t *>(q);
    A.k = static_cast<const uint16_t *>(k);
    A.v = static_cast<const uint16_t *>(v);
    A.pos = positions;
    A.qw = static_cast<const uint16_t *>(q_norm_weight);
    A.kw = static_cast<const uint16_t *>(k_norm_weight);
    A.slots = slot_mapping;
    A.q_out = static_cast<uint16_t *>(q_out);
    A.kp = static_cast<uint16_t *>(k_pool);
    A.vp = static_cast<uint16_t *>(v_pool);
    A.n = n;
    A.Hq = num_q_heads;
    A.Hkv = num_kv_heads;
    A.num_blocks = num_blocks;
    A.rotary_dim = rotary_dim;
    A.eps = eps;
    A.weight_offset = weight_offset;
    A.log2_theta = std::log2((double)rope_theta);
    hipStream_t st = reinterpret_cast<hipStream_t>(hip_stream);
    (void)hipGetLastError();
    const dim3 grid((unsigned)groups, (unsigned)hgroups);
    if (head_dim == 64) hipLaunchKernelGGL(qknorm_rope_scatter_kernel<64>, grid, dim3(256), 0, st, A);
    else if (head_dim == 128) hipLaunchKernelGGL(qknorm_rope_scatter_kernel<128>, grid, dim3(256), 0, st, A);
    else hipLaunchKernelGGL(qknorm_rope_scatter_kernel<256>, grid, dim3(256), 0, st, A);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) PKV_FAIL(KV_EDEVICE, "kv_qknorm_rope_scatter: launch failed: %s", hipGetErrorString(e));
    return KV_OK;
}

}  // extern "C"
