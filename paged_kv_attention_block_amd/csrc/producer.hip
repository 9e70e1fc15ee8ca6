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
// Workgroup: 16 consecutive tokens x up to HPW heads of one kind (Q, K or
// V): 4, or 2 when a batch is so small that 4 would leave most compute
// units idle. Lane group t (16 lanes) owns token t; lane p of it owns the D/16
// consecutive dimensions p*D/16 .. p*D/16 + D/16 - 1, held as packed bf16
// pairs, so that a row loads and stores in 16-byte pieces and the K tile
// layout [D/8][16][8] takes whole pieces. The NeoX partner of a dimension
// sits rotary_dim/2 / (D/16) lanes away, in the same register (8 lanes when
// the whole head turns: one DPP row rotation). A Q or K workgroup computes
// its 16 x rotary_dim/2 angles once, spread over all its lanes and shared
// through LDS: the angle in float64, reduced by multiples of pi/2, then
// short polynomials in float32. The norm weights fold into the rotation
// factors (w cos, and the partner's weight times the signed sine), and each
// row is rounded to bf16 once by the hardware's packed conversion (nearest,
// ties to even). A V workgroup only moves rows: whole blocks turn into the
// [D][16] tile through LDS.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <type_traits>

#include "pagedkv.h"
#include "status.h"

namespace pkv {
namespace {

constexpr int kBlk = 16;

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

struct ProdArgs {
    const uint16_t *q, *k, *v;  // [n][H][D] bf16
    const int32_t *pos;         // [n]
    const uint16_t *qw, *kw;    // [D] bf16 or null
    const int32_t *slots;       // [n]
    uint16_t *q_out;            // [n][Hq][D]
    uint16_t *kp, *vp;          // pools
    int n, Hq, Hkv, num_blocks, rotary_dim;
    float eps, weight_offset;
    double freq_step;  // 2 log2(theta) / rotary_dim: pair i turns at 2^(-i freq_step) per position
};

// A row piece is held as packed bf16 pairs: word i has dimension 2i in its
// low half and 2i + 1 in its high half.
__device__ inline float lo_f32(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ inline float hi_f32(uint32_t w) { return __builtin_bit_cast(float, w & 0xFFFF0000u); }
__device__ inline float half_f32(uint32_t w, int e) { return e & 1 ? hi_f32(w) : lo_f32(w); }

// Two floats to a bf16 pair, each rounded to the nearest, ties to even
// (one packed conversion instruction on gfx950).
__device__ inline uint32_t pack_bf16(float a, float b) {
    const f32x2_t f = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}

template <int W>
__device__ inline void load_words(const uint16_t *src, uint32_t (&x)[W]) {
    if constexpr (W == 2) {
        const u32x2_t w = *reinterpret_cast<const u32x2_t *>(src);
        x[0] = w.x;
        x[1] = w.y;
    } else {
#pragma unroll
        for (int c = 0; c < W; c += 4) {
            const u32x4_t w = *reinterpret_cast<const u32x4_t *>(src + 2 * c);
            x[c] = w.x;
            x[c + 1] = w.y;
            x[c + 2] = w.z;
            x[c + 3] = w.w;
        }
    }
}

template <int W>
__device__ inline void store_words(uint16_t *dst, const uint32_t (&x)[W]) {
    if constexpr (W == 2) {
        *reinterpret_cast<u32x2_t *>(dst) = u32x2_t{x[0], x[1]};
    } else {
#pragma unroll
        for (int c = 0; c < W; c += 4)
            *reinterpret_cast<u32x4_t *>(dst + 2 * c) = u32x4_t{x[c], x[c + 1], x[c + 2], x[c + 3]};
    }
}

// Lane (i + n) mod 16 of the lane's 16-lane row (DPP row rotation).
template <int N>
__device__ inline float row_ror(float x) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x120 + N, 0xF, 0xF, false));
}

// Sine and cosine of an angle held in float64. The angle is reduced by the
// nearest multiple q of pi/2 in float64 (one fused multiply-add with the
// double-precision pi/2), leaving |r| <= pi/4, which goes to float32; the
// Taylor series of sin r to r^9 and of cos r to r^10 are below 2e-9 from
// the exact values there, and q mod 4 picks and signs the pair:
// sin(q pi/2 + r) is sin r, cos r, -sin r, -cos r and the cosine is
// cos r, -sin r, -cos r, sin r for q = 0, 1, 2, 3 (signs set on the sign
// bit).
__device__ inline void sincos_turned(double ang, float &s, float &c) {
    const double q = rint(ang * (2.0 / M_PI));
    const float r = (float)fma(-q, M_PI_2, ang);
    const int k = (int)q;  // the quadrant is k mod 4 (two's complement keeps it for k < 0)
    const float r2 = r * r;
    float ps = fmaf(r2, 1.f / 362880.f, -1.f / 5040.f);
    ps = fmaf(ps, r2, 1.f / 120.f);
    ps = fmaf(ps, r2, -1.f / 6.f);
    const float sr = fmaf(ps * r2, r, r);
    float pc = fmaf(r2, -1.f / 3628800.f, 1.f / 40320.f);
    pc = fmaf(pc, r2, -1.f / 720.f);
    pc = fmaf(pc, r2, 1.f / 24.f);
    pc = fmaf(pc, r2, -0.5f);
    const float cr = fmaf(pc, r2, 1.f);
    const float a = (k & 1) ? cr : sr, b = (k & 1) ? sr : cr;
    s = __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, a) ^ ((uint32_t)(k & 2) << 30));
    c = __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, b) ^ ((uint32_t)((k + 1) & 2) << 30));
}

template <int D, int HPW>
__global__ __launch_bounds__(256) void qknorm_rope_scatter_kernel(ProdArgs A) {
    constexpr int CPT = D / 16, W = CPT / 2;
    const int tid = threadIdx.x;
    const int t = tid >> 4, part = tid & 15, lane = tid & 63;
    const int i0 = blockIdx.x * kBlk;
    const int tok = i0 + t;
    const bool have = tok < A.n;

    // Head groups: the Q heads HPW at a time, then the K heads, then
    // the V heads (the last group of each kind may hold fewer), so that a
    // workgroup's rows are all of one kind.
    const int gq = (A.Hq + HPW - 1) / HPW, gk = (A.Hkv + HPW - 1) / HPW;
    const int gy = blockIdx.y;
    const int kind = gy < gq ? 0 : gy < gq + gk ? 1 : 2;  // Q, K, V
    const int head0 = (kind == 0 ? gy : kind == 1 ? gy - gq : gy - gq - gk) * HPW;
    const int H = kind == 0 ? A.Hq : A.Hkv;
    const int nh = min(H - head0, HPW);

    __shared__ int s_slot[kBlk];
    __shared__ int s_pos[kBlk];
    __shared__ double s_inv_freq[D / 2];  // theta^(-2i / rotary_dim), i < rotary_dim / 2
    // Q and K workgroups: (cos, sin) of token t's pair index i, [kBlk][D/2];
    // V workgroups: their rows, [HPW][kBlk][D] bf16
    constexpr int kCsBytes = kBlk * (D / 2) * 8, kVBytes = HPW * kBlk * D * 2;
    __shared__ __attribute__((aligned(16))) unsigned char s_u[kCsBytes > kVBytes ? kCsBytes : kVBytes];
    float2(&s_cs)[kBlk][D / 2] = *reinterpret_cast<float2(*)[kBlk][D / 2]>(s_u);
    uint16_t(&sv)[HPW][kBlk][D] = *reinterpret_cast<uint16_t(*)[HPW][kBlk][D]>(s_u);

    // Every global read is issued up front, the per-token ones first, so
    // that one memory latency covers them all and the angle arithmetic
    // overlaps the row reads (indices clamped to the last token, n >= 1, so
    // that no load sits in a branch of its own; the clamped values are
    // masked below).
    const int slot_g = A.slots[min(i0 + (tid & (kBlk - 1)), A.n - 1)];
    const int pos_g = A.pos[min(i0 + (tid & (kBlk - 1)), A.n - 1)];
    const uint16_t *wsrc = kind == 0 ? A.qw : kind == 1 ? A.kw : nullptr;
    uint32_t wv[W];  // the lane's dimensions of the kind's norm weights
    if (wsrc) load_words<W>(wsrc + part * CPT, wv);
    const uint16_t *rows_in = kind == 0 ? A.q : kind == 1 ? A.k : A.v;
    uint32_t xs[HPW][W];
#pragma unroll
    for (int j = 0; j < HPW; ++j)
        load_words<W>(rows_in + ((size_t)(have ? tok : 0) * H + head0 + min(j, nh - 1)) * D + part * CPT, xs[j]);
    if (tid < kBlk) s_slot[tid] = (i0 + tid < A.n && slot_g >= 0 && slot_g < A.num_blocks * kBlk) ? slot_g : -1;

    if (kind == 2) {
        // V rows go into the pools unchanged. Tile [D][16]: when the 16
        // tokens fill one block in order, the rows turn through LDS and
        // leave in 16-byte pieces of 8 tokens; otherwise value by value.
        __syncthreads();
        const int slot = s_slot[t];
        const int sl0 = s_slot[0];
        const int li = lane & (kBlk - 1);
        const bool full = __all(lane >= kBlk || (s_slot[li] >= 0 && s_slot[li] == sl0 + li && sl0 % kBlk == 0));
        if (full) {
#pragma unroll
            for (int j = 0; j < HPW; ++j)
                if (j < nh) store_words<W>(&sv[j][t][part * CPT], xs[j]);
            __syncthreads();
            for (int pc = tid; pc < nh * 2 * D; pc += 256) {  // row j, piece q: channel q/2, tokens 8 (q&1) .. +7
                const int j = pc / (2 * D), q = pc - j * 2 * D;
                const int c = q >> 1, t0 = (q & 1) * 8;
                uint32_t b[4];
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    b[e] = (uint32_t)sv[j][t0 + 2 * e][c] | ((uint32_t)sv[j][t0 + 2 * e + 1][c] << 16);
                uint16_t *tile = A.vp + ((size_t)(sl0 / kBlk) * A.Hkv + head0 + j) * kBlk * D;
                *reinterpret_cast<u32x4_t *>(tile + (size_t)q * 8) = u32x4_t{b[0], b[1], b[2], b[3]};
            }
        } else if (have && slot >= 0) {
#pragma unroll
            for (int j = 0; j < HPW; ++j) {
                if (j >= nh) break;
                uint16_t *tile = A.vp + ((size_t)(slot / kBlk) * A.Hkv + head0 + j) * kBlk * D;
#pragma unroll
                for (int e = 0; e < CPT; ++e)
                    tile[(size_t)(part * CPT + e) * kBlk + slot % kBlk] =
                        (uint16_t)(e & 1 ? xs[j][e / 2] >> 16 : xs[j][e / 2] & 0xFFFFu);
            }
        }
        return;
    }

    const int half = A.rotary_dim / 2;
    const int shift = half / CPT;  // lanes between NeoX partners; 8 when the whole head turns
    if (tid < half) s_inv_freq[tid] = exp2(-(double)tid * A.freq_step);
    if (tid < kBlk) s_pos[tid] = i0 + tid < A.n ? pos_g : 0;
    __syncthreads();
    // the workgroup's 16 x rotary_dim/2 angles, once each, over all lanes;
    // when rotary_dim/2 is a power of two a lane keeps one pair index and
    // steps over the tokens
    if (half > 0 && (half & (half - 1)) == 0) {
        const int lg = __builtin_ctz(half);
        const int i = tid & (half - 1);
        const double f = s_inv_freq[i];
        for (int tt = tid >> lg; tt < kBlk; tt += 256 >> lg) {
            float sv_, cv;
            sincos_turned((double)s_pos[tt] * f, sv_, cv);
            s_cs[tt][i] = make_float2(cv, sv_);
        }
    } else {
        for (int idx = tid; idx < kBlk * half; idx += 256) {
            const int tt = idx / half, i = idx - tt * half;
            float sv_, cv;
            sincos_turned((double)s_pos[tt] * s_inv_freq[i], sv_, cv);
            s_cs[tt][i] = make_float2(cv, sv_);
        }
    }
    __syncthreads();
    const int slot = s_slot[t];
    const bool lower = part * CPT < half;
    const int src_lane = lower ? lane + shift : lane - shift;

    // A row value and its partner's, normalized (xh = x inv) and weighted,
    // turn into xh w cos + xh' w' sin, w' the partner dimension's weight and
    // the sine signed for the pair member (the lower member takes minus its
    // partner's share, the upper plus). Both factors are formed once:
    // fa = w cos, fb = w' sin. Dimension c < rotary_dim turns by the angle
    // of pair index c mod rotary_dim/2; past rotary_dim, cos 1 and sin 0.
    float fa[CPT], fb[CPT];
    {
        const int base = lower ? part * CPT : part * CPT - half;
#pragma unroll
        for (int e = 0; e < CPT; ++e) {
            const float w = wsrc ? A.weight_offset + half_f32(wv[e / 2], e) : 1.f;
            const bool rot = part * CPT + e < A.rotary_dim;
            const float2 v = rot ? s_cs[t][base + e] : make_float2(1.f, 0.f);
            const float wp = shift == 8 ? row_ror<8>(w) : __shfl(w, shift ? src_lane : lane, 64);
            fa[e] = w * v.x;
            fb[e] = wp * (lower ? -v.y : v.y);
        }
    }

    // norm and rotation of each row, stored as soon as it is done
    auto rows = [&](auto dpp) {
        constexpr bool DPP = decltype(dpp)::value;  // the whole head turns: partners 8 lanes apart
#pragma unroll
        for (int j = 0; j < HPW; ++j) {
            if (j >= nh) break;  // uniform over the workgroup
            const int head = head0 + j;
            uint32_t(&x)[W] = xs[j];
            float ss = 0.f;
#pragma unroll
            for (int e = 0; e < CPT; ++e) {
                const float y = half_f32(x[e / 2], e);
                ss = fmaf(y, y, ss);
            }
            // sum over the token's 16 lanes: after the step by n, lanes n
            // apart hold equal sums, so a rotation by n adds the same pair as
            // an exchange with lane i ^ n
            ss += row_ror<8>(ss);
            ss += row_ror<4>(ss);
            ss += row_ror<2>(ss);
            ss += row_ror<1>(ss);
            const float inv = __frsqrt_rn(ss * (1.f / D) + A.eps);  // D a power of two: the mean is exact
            float xh[CPT], r[CPT];
#pragma unroll
            for (int e = 0; e < CPT; ++e) xh[e] = half_f32(x[e / 2], e) * inv;
#pragma unroll
            for (int e = 0; e < CPT; ++e) {
                const float other = DPP ? row_ror<8>(xh[e]) : __shfl(xh[e], shift ? src_lane : lane, 64);
                const float own = xh[e] * fa[e];  // xh w where the dimension does not turn
                r[e] = DPP || part * CPT + e < A.rotary_dim ? fmaf(other, fb[e], own) : own;
            }
#pragma unroll
            for (int i = 0; i < W; ++i) x[i] = pack_bf16(r[2 * i], r[2 * i + 1]);
            if (kind == 0) {
                if (have) store_words<W>(A.q_out + ((size_t)tok * A.Hq + head) * D + part * CPT, x);
            } else if (have && slot >= 0) {
                // K tile [D/8][16][8]: the lane's dimensions are whole 8-element pieces
                uint16_t *tile = A.kp + ((size_t)(slot / kBlk) * A.Hkv + head) * kBlk * D;
                const int o = slot % kBlk;
#pragma unroll
                for (int i = 0; i < W; i += 4 < W ? 4 : W) {
                    const int c0 = part * CPT + 2 * i;
                    uint16_t *dst = tile + ((c0 / 8) * kBlk + o) * 8 + c0 % 8;
                    if constexpr (W == 2) *reinterpret_cast<u32x2_t *>(dst) = u32x2_t{x[i], x[i + 1]};
                    else *reinterpret_cast<u32x4_t *>(dst) = u32x4_t{x[i], x[i + 1], x[i + 2], x[i + 3]};
                }
            }
        }
    };
    if (shift == 8) rows(std::true_type{});
    else rows(std::false_type{});
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
    // head groups of `hpw` heads per kind; 2 when 4 would give fewer than
    // 128 workgroups (decode-sized batches, where latency rules)
    auto head_groups = [&](int64_t hpw) {
        return (num_q_heads + hpw - 1) / hpw + 2 * ((num_kv_heads + hpw - 1) / hpw);
    };
    const int hpw = groups * head_groups(4) < 128 ? 2 : 4;
    const int64_t hgroups = head_groups(hpw);
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
    A.freq_step = rotary_dim ? 2.0 * std::log2((double)rope_theta) / rotary_dim : 0.0;
    hipStream_t st = reinterpret_cast<hipStream_t>(hip_stream);
    (void)hipGetLastError();
    const dim3 grid((unsigned)groups, (unsigned)hgroups);
    auto launch = [&](auto kernel) { hipLaunchKernelGGL(kernel, grid, dim3(256), 0, st, A); };
    if (head_dim == 64) hpw == 2 ? launch(qknorm_rope_scatter_kernel<64, 2>) : launch(qknorm_rope_scatter_kernel<64, 4>);
    else if (head_dim == 128)
        hpw == 2 ? launch(qknorm_rope_scatter_kernel<128, 2>) : launch(qknorm_rope_scatter_kernel<128, 4>);
    else hpw == 2 ? launch(qknorm_rope_scatter_kernel<256, 2>) : launch(qknorm_rope_scatter_kernel<256, 4>);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) PKV_FAIL(KV_EDEVICE, "kv_qknorm_rope_scatter: launch failed: %s", hipGetErrorString(e));
    return KV_OK;
}

}  // extern "C"
