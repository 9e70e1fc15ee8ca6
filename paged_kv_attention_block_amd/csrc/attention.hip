// Batched attention over a paged KV cache, and the paged K/V scatter-write,
// for gfx950 (CDNA4, wave64).
//
// TensorSharp "高级功能" page, section "原生分页注意力": one native call gathers
// K/V through the paged buffers for many sequences and runs fused attention,
// with a variant taking per-head sink logits; its "批量前向" paragraph pairs the
// batched forward with a paged K/V scatter-write. Decode rows, chunked-prefill
// rows (section "性能优化", chunked prefill) and speculative-verify windows
// (section "MTP / NextN 推测解码") share one entry point. The speculative-
// decoding pages (the TensorFold sections on the exactness rule and on
// row-invariant wide-window kernels) require that a row computed alone and
// the same row inside a window give identical bits; every design choice below
// that fixes an order of floating-point operations exists for that.
//
// Arithmetic of one (query row, query head), identical for every row whatever
// the batch, window or q_len around it:
//  * keys are cut into splits by a fixed function of absolute key position
//    (split_begin); one wave owns one split of one (sequence, KV head, rows);
//  * inside a split, keys are consumed in 32-key chunks (two 16-token blocks)
//    in ascending order with an online softmax in base 2;
//  * bf16: S^T = K * Q^T and O^T = V^T * P^T on 16x16x32 bf16 MFMA tiles whose
//    results were measured to be independent of the row's position in the
//    tile; P enters the PV product as a hi + lo pair of bf16 values;
//  * fp32: plain fp32 FMA chains, one wave per (row, head);
//  * a separate pass folds the splits of each (row, head) left to right, adds
//    the sink term and divides once.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "pagedkv.h"
#include "status.h"

namespace pkv {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kBlock = 16;
constexpr int kChunk = 32;
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kMaxHeadDim = 128;

// ---------------------------------------------------------------------------
// Fixed split partition of absolute key positions:
//   [0, 1024)    64-key splits   (indices 0..15)
//   [1024, 4096) 256-key splits  (indices 16..27)
//   [4096, ...)  512-key splits  (indices 28..)
// Small splits near the start give short contexts enough waves; long splits
// further out keep the partial results small next to the K/V they summarise.
// ---------------------------------------------------------------------------
__host__ __device__ inline int split_index(int pos) {
    if (pos < 1024) return pos >> 6;
    if (pos < 4096) return 16 + ((pos - 1024) >> 8);
    return 28 + ((pos - 4096) >> 9);
}
__host__ __device__ inline int split_begin(int idx) {
    if (idx < 16) return idx << 6;
    if (idx < 28) return 1024 + ((idx - 16) << 8);
    return 4096 + ((idx - 28) << 9);
}
__host__ __device__ inline int num_splits(int len) { return len <= 0 ? 0 : split_index(len - 1) + 1; }

struct AttnParams {
    const void *q;
    const void *kp;
    const void *vp;
    const int32_t *bt;
    const int32_t *ctx_lens;
    const int32_t *qsl;
    const float *sinks;
    float2 *ws_ml;   // [rows][Hq][max_splits] (running max in log2 units, sum)
    float *ws_acc;   // [rows][Hq][max_splits][D]
    float *out;      // [rows][Hq][D]
    int32_t num_seqs, total_rows, Hq, Hkv, G, max_blocks_per_seq, num_blocks, max_splits;
    float scale_log2;
};

// A zero (block, head) tile: loads of blocks past the end of a sequence read it.
__device__ __attribute__((aligned(16))) uint16_t g_zero_tile[kBlock * kMaxHeadDim];

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ inline int seq_of_row(const int32_t *qsl, int num_seqs, int row) {
    int lo = 0, hi = num_seqs;  // qsl[lo] <= row < qsl[hi]
    while (hi - lo > 1) {
        int mid = (lo + hi) >> 1;
        if (qsl[mid] <= row) lo = mid; else hi = mid;
    }
    return lo;
}

// ---------------------------------------------------------------------------
// bf16 split kernel. One wave: (sequence s, KV head, rows row0..row0+16*NT-1
// of the s-th [q_len * G] row space ordered as r * G + head_in_group, one split).
// Lane l = 16 g + n: n is the MFMA column (query row of the tile), g the
// k-slot group.
// ---------------------------------------------------------------------------
template <int D>
struct ChunkRegs {
    u32x4_t k[2][D / 32];   // A operand of S^T = K Q^T, per block tau and k-step j
    u32x2_t v[2][D / 16];   // half of the A operand of O^T = V^T P^T, per block and d-tile
};

template <int D>
__device__ inline void load_chunk(ChunkRegs<D> &c, const uint16_t *kb0, const uint16_t *vb0,
                                  const uint16_t *kb1, const uint16_t *vb1, int g, int n) {
#pragma unroll
    for (int j = 0; j < D / 32; ++j) {
        c.k[0][j] = *reinterpret_cast<const u32x4_t *>(kb0 + ((4 * j + g) * kBlock + n) * 8);
        c.k[1][j] = *reinterpret_cast<const u32x4_t *>(kb1 + ((4 * j + g) * kBlock + n) * 8);
    }
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
        c.v[0][dt] = *reinterpret_cast<const u32x2_t *>(vb0 + (16 * dt + n) * kBlock + 4 * g);
        c.v[1][dt] = *reinterpret_cast<const u32x2_t *>(vb1 + (16 * dt + n) * kBlock + 4 * g);
    }
}

template <int D, int NT>
__global__ __launch_bounds__(64) void attn_bf16_split(AttnParams P, int one_item_per_seq) {
    constexpr int R = 16 * NT;
    constexpr int KJ = D / 32;
    constexpr int DT = D / 16;
    const int lane = threadIdx.x;
    const int g = lane >> 4, n = lane & 15;
    const int item = blockIdx.x, kvh = blockIdx.y, split = blockIdx.z;

    int s = 0, rb = 0;
    if (one_item_per_seq) {
        s = item;
        if (s >= P.num_seqs) return;
    } else {
        int acc = 0;
        bool found = false;
        for (int t = 0; t < P.num_seqs; ++t) {
            const int nb = ((P.qsl[t + 1] - P.qsl[t]) * P.G + R - 1) / R;
            if (item < acc + nb) { s = t; rb = item - acc; found = true; break; }
            acc += nb;
        }
        if (!found) return;
    }
    const int q0 = P.qsl[s];
    const int q_len = P.qsl[s + 1] - q0;
    const int ctx = P.ctx_lens[s];
    if (q0 < 0 || q_len <= 0 || q0 + q_len > P.total_rows) return;
    const int rows_total = q_len * P.G;
    const int row0 = rb * R;
    if (row0 >= rows_total) return;
    const int row_last = min(row0 + R, rows_total) - 1;
    const int p_max = ctx - q_len + row_last / P.G;
    const int ks = split_begin(split);
    if (ks > p_max) return;
    const int ke = min(split_begin(split + 1), p_max + 1);

    // Rows of this lane (column n of every tile) and the Q operand.
    int prow[NT];
    u32x4_t qop[NT][KJ];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        const int rho = row0 + t * 16 + n;
        const int r = rho / P.G;
        const bool valid = rho < rows_total && q0 + r < P.total_rows;
        const int rr = valid ? r : 0;                    // keep the address in bounds
        const int hl = valid ? rho - r * P.G : 0;
        prow[t] = valid ? ctx - q_len + r : -1;
        const uint16_t *qrow = reinterpret_cast<const uint16_t *>(P.q) +
                               ((size_t)(q0 + rr) * P.Hq + kvh * P.G + hl) * D;
#pragma unroll
        for (int j = 0; j < KJ; ++j)
            qop[t][j] = valid ? *reinterpret_cast<const u32x4_t *>(qrow + 32 * j + 8 * g)
                              : u32x4_t{0, 0, 0, 0};
    }

    // Physical block ids of the split, one per lane.
    const int jb0 = ks / kBlock;
    const int nblk_seq = (ctx + kBlock - 1) / kBlock;
    const int nb_split = (ke - ks + kBlock - 1) / kBlock;
    int bid = -1;
    if (lane < nb_split) {
        const int jb = jb0 + lane;
        if (jb < nblk_seq && jb < P.max_blocks_per_seq) {
            const int b = P.bt[(size_t)s * P.max_blocks_per_seq + jb];
            bid = (b >= 0 && b < P.num_blocks) ? b : -1;
        }
    }
    const size_t tile = (size_t)kBlock * D;
    const uint16_t *kbase = reinterpret_cast<const uint16_t *>(P.kp) + (size_t)kvh * tile;
    const uint16_t *vbase = reinterpret_cast<const uint16_t *>(P.vp) + (size_t)kvh * tile;
    const size_t bstride = (size_t)P.Hkv * tile;
    auto kptr = [&](int b) { return b >= 0 ? kbase + (size_t)b * bstride : g_zero_tile; };
    auto vptr = [&](int b) { return b >= 0 ? vbase + (size_t)b * bstride : g_zero_tile; };

    float m[NT], l[NT];
    f32x4_t acc[NT][DT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        m[t] = -INFINITY;
        l[t] = 0.f;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) acc[t][dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }

    auto compute = [&](ChunkRegs<D> &c, int kc) {
        if (kc + kChunk > ctx) {
            // keys at or past ctx: zero V so that weight 0 never meets a NaN
#pragma unroll
            for (int tau = 0; tau < 2; ++tau) {
                const int k0 = kc + 16 * tau + 4 * g;
                const uint32_t m0 = (k0 < ctx ? 0x0000FFFFu : 0u) | (k0 + 1 < ctx ? 0xFFFF0000u : 0u);
                const uint32_t m1 = (k0 + 2 < ctx ? 0x0000FFFFu : 0u) | (k0 + 3 < ctx ? 0xFFFF0000u : 0u);
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) {
                    c.v[tau][dt].x &= m0;
                    c.v[tau][dt].y &= m1;
                }
            }
        }
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            if (row0 + t * 16 >= rows_total) continue;
            f32x4_t s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < KJ; ++j) {
                const bf16x8_t b = __builtin_bit_cast(bf16x8_t, qop[t][j]);
                s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, c.k[0][j]), b, s0, 0, 0, 0);
                s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, c.k[1][j]), b, s1, 0, 0, 0);
            }
            float sc[8];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int key = kc + 4 * g + i;
                sc[i] = key <= prow[t] ? s0[i] * P.scale_log2 : -INFINITY;
                sc[4 + i] = key + 16 <= prow[t] ? s1[i] * P.scale_log2 : -INFINITY;
            }
            float mx = sc[0];
#pragma unroll
            for (int e = 1; e < 8; ++e) mx = fmaxf(mx, sc[e]);
            mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
            mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
            const float m_new = fmaxf(m[t], mx);
            const float m_use = m_new == -INFINITY ? 0.f : m_new;
            const float alpha = fast_exp2(m[t] - m_use);
            float pv[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) pv[e] = fast_exp2(sc[e] - m_use);
            float rs = pv[0];
#pragma unroll
            for (int e = 1; e < 8; ++e) rs += pv[e];
            rs += __shfl_xor(rs, 16, 64);
            rs += __shfl_xor(rs, 32, 64);
            l[t] = alpha * l[t] + rs;
            m[t] = m_new;
            bf16x8_t phi, plo;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const __bf16 h = (__bf16)pv[e];
                phi[e] = h;
                plo[e] = (__bf16)(pv[e] - (float)h);
            }
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                const u32x4_t va4 = {c.v[0][dt].x, c.v[0][dt].y, c.v[1][dt].x, c.v[1][dt].y};
                const bf16x8_t va = __builtin_bit_cast(bf16x8_t, va4);
                f32x4_t a = acc[t][dt] * alpha;
                a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, plo, a, 0, 0, 0);
                acc[t][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, phi, a, 0, 0, 0);
            }
        }
    };

    // Two register sets: the next chunk's loads are in flight while the
    // current chunk is computed.
    ChunkRegs<D> ca, cb;
    {
        const int b0 = __builtin_amdgcn_readlane(bid, 0);
        const int b1 = __builtin_amdgcn_readlane(bid, 1);
        load_chunk<D>(ca, kptr(b0), vptr(b0), kptr(b1), vptr(b1), g, n);
    }
    for (int kc = ks; kc < ke; kc += 2 * kChunk) {
        const bool has_b = kc + kChunk < ke;
        if (has_b) {
            const int ci = (kc + kChunk - ks) / kBlock;
            const int b0 = __builtin_amdgcn_readlane(bid, ci);
            const int b1 = __builtin_amdgcn_readlane(bid, ci + 1);
            load_chunk<D>(cb, kptr(b0), vptr(b0), kptr(b1), vptr(b1), g, n);
        }
        compute(ca, kc);
        if (!has_b) break;
        if (kc + 2 * kChunk < ke) {
            const int ci = (kc + 2 * kChunk - ks) / kBlock;
            const int b0 = __builtin_amdgcn_readlane(bid, ci);
            const int b1 = __builtin_amdgcn_readlane(bid, ci + 1);
            load_chunk<D>(ca, kptr(b0), vptr(b0), kptr(b1), vptr(b1), g, n);
        }
        compute(cb, kc + kChunk);
    }

    // Partial results of this split for rows that see at least one of its keys.
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        if (prow[t] < ks) continue;
        const int rho = row0 + t * 16 + n;
        const int r = rho / P.G;
        const int hl = rho - r * P.G;
        const size_t base = ((size_t)(q0 + r) * P.Hq + kvh * P.G + hl) * P.max_splits + split;
        if (g == 0) P.ws_ml[base] = make_float2(m[t], l[t]);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
            *reinterpret_cast<f32x4_t *>(P.ws_acc + base * D + 16 * dt + 4 * g) = acc[t][dt];
    }
}

// ---------------------------------------------------------------------------
// fp32 split kernel: one wave per (row, query head, split); lane t takes key
// kc + t of each 64-key chunk for the scores and channel d = lane (+64) for
// the value sum.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(64) void attn_f32_split(AttnParams P) {
    constexpr int DU = D / 64;
    const int lane = threadIdx.x;
    const int i = blockIdx.x, h = blockIdx.y, split = blockIdx.z;
    const int s = seq_of_row(P.qsl, P.num_seqs, i);
    const int q_len = P.qsl[s + 1] - P.qsl[s];
    const int ctx = P.ctx_lens[s];
    const int p = ctx - q_len + (i - P.qsl[s]);
    const int ks = split_begin(split);
    if (ks > p) return;
    const int ke = min(split_begin(split + 1), p + 1);
    const int kvh = h / P.G;

    __shared__ float qs[D];
    const float *qrow = reinterpret_cast<const float *>(P.q) + ((size_t)i * P.Hq + h) * D;
#pragma unroll
    for (int u = 0; u < DU; ++u) qs[lane + 64 * u] = qrow[lane + 64 * u];
    __syncthreads();

    const float *kp = reinterpret_cast<const float *>(P.kp);
    const float *vp = reinterpret_cast<const float *>(P.vp);
    const size_t tile = (size_t)kBlock * D;
    float m = -INFINITY, l = 0.f;
    float acc[DU];
#pragma unroll
    for (int u = 0; u < DU; ++u) acc[u] = 0.f;

    for (int kc = ks; kc < ke; kc += 64) {
        const int key = kc + lane;
        const bool vis = key < ke;
        int phys = -1;
        if (vis) {
            const int jb = key / kBlock;
            if (jb < P.max_blocks_per_seq) {
                const int b = P.bt[(size_t)s * P.max_blocks_per_seq + jb];
                phys = (b >= 0 && b < P.num_blocks) ? b : -1;
            }
        }
        float dot = 0.f;
        if (phys >= 0) {
            const float *kb = kp + ((size_t)phys * P.Hkv + kvh) * tile;
            const int o = key % kBlock;
#pragma unroll
            for (int c = 0; c < D / 4; ++c) {
                const f32x4_t kv = *reinterpret_cast<const f32x4_t *>(kb + (c * kBlock + o) * 4);
                dot = fmaf(qs[4 * c + 0], kv[0], dot);
                dot = fmaf(qs[4 * c + 1], kv[1], dot);
                dot = fmaf(qs[4 * c + 2], kv[2], dot);
                dot = fmaf(qs[4 * c + 3], kv[3], dot);
            }
        }
        const float sc = vis ? dot * P.scale_log2 : -INFINITY;
        float mx = sc;
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
        const float m_new = fmaxf(m, mx);
        const float m_use = m_new == -INFINITY ? 0.f : m_new;
        const float alpha = fast_exp2(m - m_use);
        const float pv = fast_exp2(sc - m_use);
        float rs = pv;
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) rs += __shfl_xor(rs, o, 64);
        l = alpha * l + rs;
        m = m_new;
#pragma unroll
        for (int u = 0; u < DU; ++u) acc[u] *= alpha;
        for (int bb = 0; bb < 4; ++bb) {
            const int kb0 = kc + kBlock * bb;
            if (kb0 >= ke) break;
            const int pb = __builtin_amdgcn_readlane(phys, kBlock * bb);
            if (pb < 0) continue;
#pragma unroll
            for (int u = 0; u < DU; ++u) {
                const float *vrow = vp + ((size_t)pb * P.Hkv + kvh) * tile + (size_t)(lane + 64 * u) * kBlock;
                float vv[kBlock];
#pragma unroll
                for (int q4 = 0; q4 < kBlock / 4; ++q4) {
                    const f32x4_t x = *reinterpret_cast<const f32x4_t *>(vrow + 4 * q4);
                    vv[4 * q4 + 0] = x[0];
                    vv[4 * q4 + 1] = x[1];
                    vv[4 * q4 + 2] = x[2];
                    vv[4 * q4 + 3] = x[3];
                }
#pragma unroll
                for (int tt = 0; tt < kBlock; ++tt) {
                    const float w = __builtin_bit_cast(
                        float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, pv), kBlock * bb + tt));
                    const float v = kb0 + tt < ke ? vv[tt] : 0.f;
                    acc[u] = fmaf(w, v, acc[u]);
                }
            }
        }
    }
    const size_t base = ((size_t)i * P.Hq + h) * P.max_splits + split;
    if (lane == 0) P.ws_ml[base] = make_float2(m, l);
#pragma unroll
    for (int u = 0; u < DU; ++u) P.ws_acc[base * D + lane + 64 * u] = acc[u];
}

// ---------------------------------------------------------------------------
// Split fold: one wave per (row, query head); lanes own channels.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(64) void attn_reduce(AttnParams P) {
    constexpr int DU = D / 64;
    const int lane = threadIdx.x;
    const int i = blockIdx.x, h = blockIdx.y;
    const int s = seq_of_row(P.qsl, P.num_seqs, i);
    const int q_len = P.qsl[s + 1] - P.qsl[s];
    const int ctx = P.ctx_lens[s];
    const int p = ctx - q_len + (i - P.qsl[s]);
    const int ns = min(num_splits(p + 1), P.max_splits);
    const size_t base = ((size_t)i * P.Hq + h) * P.max_splits;
    // split maxima and sums, one split per lane (64 at a time), loaded together
    float M = -INFINITY;
    for (int j0 = 0; j0 < ns; j0 += 64) {
        const float mj = j0 + lane < ns ? P.ws_ml[base + j0 + lane].x : -INFINITY;
        M = fmaxf(M, mj);
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o, 64));
    const float sk = P.sinks ? P.sinks[h] * kLog2e : -INFINITY;
    M = fmaxf(M, sk);
    float L = 0.f;
    float a[DU];
#pragma unroll
    for (int u = 0; u < DU; ++u) a[u] = 0.f;
    for (int j0 = 0; j0 < ns; j0 += 64) {
        const float2 mlj = j0 + lane < ns ? P.ws_ml[base + j0 + lane] : make_float2(-INFINITY, 0.f);
        const float wj = fast_exp2(mlj.x - M);
        const int nj = min(64, ns - j0);
        int j = 0;
        for (; j + 4 <= nj; j += 4) {
            float x[4][DU];
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int u = 0; u < DU; ++u) x[t][u] = P.ws_acc[(base + j0 + j + t) * D + lane + 64 * u];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const float w = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wj), j + t));
                const float lj = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, mlj.y), j + t));
                L = fmaf(lj, w, L);
#pragma unroll
                for (int u = 0; u < DU; ++u) a[u] = fmaf(w, x[t][u], a[u]);
            }
        }
        for (; j < nj; ++j) {
            const float w = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wj), j));
            const float lj = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, mlj.y), j));
            L = fmaf(lj, w, L);
#pragma unroll
            for (int u = 0; u < DU; ++u) a[u] = fmaf(w, P.ws_acc[(base + j0 + j) * D + lane + 64 * u], a[u]);
        }
    }
    if (P.sinks) L += fast_exp2(sk - M);
#pragma unroll
    for (int u = 0; u < DU; ++u) P.out[((size_t)i * P.Hq + h) * D + lane + 64 * u] = a[u] / L;
}

// ---------------------------------------------------------------------------
// Scatter-write: one thread per (token, KV head, 16-byte piece of the head dim).
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void scatter_kernel(const T *__restrict__ kn, const T *__restrict__ vn,
                                                     const int32_t *__restrict__ slots, int n, T *kp, T *vp,
                                                     int num_blocks, int Hkv, int D) {
    constexpr int X = 16 / sizeof(T);
    const int cpt = D / X;
    const long idx = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (long)n * Hkv * cpt) return;
    const int c = (int)(idx % cpt);
    const int h = (int)((idx / cpt) % Hkv);
    const int i = (int)(idx / ((long)cpt * Hkv));
    const int slot = slots[i];
    if (slot < 0 || slot >= num_blocks * kBlock) return;
    const int b = slot / kBlock, o = slot % kBlock;
    const size_t src = ((size_t)i * Hkv + h) * D + (size_t)c * X;
    const u32x4_t kv = *reinterpret_cast<const u32x4_t *>(kn + src);
    *reinterpret_cast<u32x4_t *>(kp + ((((size_t)b * Hkv + h) * cpt + c) * kBlock + o) * X) = kv;
    const u32x4_t vv = *reinterpret_cast<const u32x4_t *>(vn + src);
    T e[X];
    __builtin_memcpy(e, &vv, 16);
    T *vd = vp + (((size_t)b * Hkv + h) * D + (size_t)c * X) * kBlock + o;
#pragma unroll
    for (int x = 0; x < X; ++x) vd[(size_t)x * kBlock] = e[x];
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
struct WsLayout {
    size_t ml_bytes, acc_bytes;
};

static WsLayout ws_layout(int64_t rows, int64_t Hq, int64_t D, int64_t splits) {
    const int64_t cells = rows * Hq * splits;
    WsLayout w;
    w.ml_bytes = (size_t)((cells * 8 + 255) / 256 * 256);
    w.acc_bytes = (size_t)(cells * D * 4);
    return w;
}

static bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

template <int D, int NT>
static void launch_bf16(const AttnParams &P, int items, int one, hipStream_t st) {
    dim3 grid(items, P.Hkv, P.max_splits);
    hipLaunchKernelGGL((attn_bf16_split<D, NT>), grid, dim3(64), 0, st, P, one);
}

template <int D>
static void launch_bf16_nt(const AttnParams &P, int max_q_len, int total_rows, hipStream_t st) {
    const int rows_per_seq = max_q_len * P.G;
    const int NT = rows_per_seq <= 16 ? 1 : (rows_per_seq <= 32 ? 2 : 4);
    const int R = 16 * NT;
    const int one = rows_per_seq <= R;
    const int items = one ? P.num_seqs : (int)(((int64_t)total_rows * P.G + R - 1) / R + P.num_seqs);
    if (NT == 1) launch_bf16<D, 1>(P, items, one, st);
    else if (NT == 2) launch_bf16<D, 2>(P, items, one, st);
    else launch_bf16<D, 4>(P, items, one, st);
}

}  // namespace pkv

extern "C" {

size_t paged_attention_workspace_size(int32_t num_seqs, int32_t total_q_rows, int32_t num_q_heads,
                                      int32_t head_dim, int32_t max_context_len) {
    if (num_seqs < 0 || total_q_rows < 0 || num_q_heads <= 0 || head_dim <= 0 || max_context_len < 0)
        return 0;
    const pkv::WsLayout w = pkv::ws_layout(total_q_rows, num_q_heads, head_dim, pkv::num_splits(max_context_len));
    return w.ml_bytes + w.acc_bytes;
}

int paged_attention_forward(const void *q, const void *k_pool, const void *v_pool, int32_t dtype,
                            const int32_t *block_tables, int32_t max_blocks_per_seq,
                            const int32_t *context_lens, const int32_t *query_start_loc,
                            int32_t num_seqs, int32_t total_q_rows, int32_t max_q_len,
                            int32_t max_context_len, int32_t num_q_heads, int32_t num_kv_heads,
                            int32_t head_dim, int32_t block_size, int32_t num_blocks, float scale,
                            const float *sinks, float *out, void *workspace, size_t workspace_bytes,
                            void *hip_stream) {
    using namespace pkv;
    if (dtype != KV_BF16 && dtype != KV_F32)
        PKV_FAIL(KV_EUNSUPPORTED, "paged_attention_forward: dtype %d not supported", dtype);
    if (head_dim != 64 && head_dim != 128)
        PKV_FAIL(KV_EUNSUPPORTED, "paged_attention_forward: head_dim %d not supported (64, 128)", head_dim);
    if (block_size != kBlock)
        PKV_FAIL(KV_EUNSUPPORTED, "paged_attention_forward: block_size %d not supported (16)", block_size);
    if (num_seqs < 0 || total_q_rows < 0 || max_q_len < 0 || max_context_len < 0 || num_blocks < 0)
        PKV_FAIL(KV_EINVAL, "paged_attention_forward: negative size");
    if (num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads)
        PKV_FAIL(KV_EINVAL, "paged_attention_forward: num_q_heads %d is not a positive multiple of num_kv_heads %d",
                 num_q_heads, num_kv_heads);
    if (num_q_heads > 65535 || num_kv_heads > 65535)
        PKV_FAIL(KV_EINVAL, "paged_attention_forward: too many heads");
    if (!std::isfinite(scale)) PKV_FAIL(KV_EINVAL, "paged_attention_forward: scale is not finite");
    if (num_seqs == 0 || total_q_rows == 0) return KV_OK;
    if (max_q_len < 1 || max_context_len < 1)
        PKV_FAIL(KV_EINVAL, "paged_attention_forward: max_q_len and max_context_len must be >= 1");
    if (max_q_len > max_context_len || max_q_len > total_q_rows)
        PKV_FAIL(KV_EINVAL, "paged_attention_forward: max_q_len %d exceeds max_context_len or total_q_rows",
                 max_q_len);
    if ((int64_t)max_blocks_per_seq * kBlock < max_context_len)
        PKV_FAIL(KV_EINVAL, "paged_attention_forward: max_blocks_per_seq %d cannot hold max_context_len %d",
                 max_blocks_per_seq, max_context_len);
    if (!q || !k_pool || !v_pool || !block_tables || !context_lens || !query_start_loc || !out || !workspace)
        PKV_FAIL(KV_EINVAL, "paged_attention_forward: required pointer is NULL");
    if (!aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool) || !aligned16(out) || !aligned16(workspace))
        PKV_FAIL(KV_EINVAL, "paged_attention_forward: q, pools, out and workspace must be 16-byte aligned");
    const int max_splits = num_splits(max_context_len);
    if (max_splits > 65535) PKV_FAIL(KV_EINVAL, "paged_attention_forward: max_context_len too large");
    const WsLayout w = ws_layout(total_q_rows, num_q_heads, head_dim, max_splits);
    if (workspace_bytes < w.ml_bytes + w.acc_bytes)
        PKV_FAIL(KV_EINVAL, "paged_attention_forward: workspace of %zu bytes, need %zu", workspace_bytes,
                 w.ml_bytes + w.acc_bytes);

    AttnParams P;
    P.q = q;
    P.kp = k_pool;
    P.vp = v_pool;
    P.bt = block_tables;
    P.ctx_lens = context_lens;
    P.qsl = query_start_loc;
    P.sinks = sinks;
    P.ws_ml = reinterpret_cast<float2 *>(workspace);
    P.ws_acc = reinterpret_cast<float *>(reinterpret_cast<char *>(workspace) + w.ml_bytes);
    P.out = out;
    P.num_seqs = num_seqs;
    P.total_rows = total_q_rows;
    P.Hq = num_q_heads;
    P.Hkv = num_kv_heads;
    P.G = num_q_heads / num_kv_heads;
    P.max_blocks_per_seq = max_blocks_per_seq;
    P.num_blocks = num_blocks;
    P.max_splits = max_splits;
    P.scale_log2 = scale * kLog2e;
    hipStream_t st = reinterpret_cast<hipStream_t>(hip_stream);

    (void)hipGetLastError();
    if (dtype == KV_BF16) {
        if (head_dim == 64) launch_bf16_nt<64>(P, max_q_len, total_q_rows, st);
        else launch_bf16_nt<128>(P, max_q_len, total_q_rows, st);
    } else {
        dim3 grid(total_q_rows, num_q_heads, max_splits);
        if (head_dim == 64) hipLaunchKernelGGL((attn_f32_split<64>), grid, dim3(64), 0, st, P);
        else hipLaunchKernelGGL((attn_f32_split<128>), grid, dim3(64), 0, st, P);
    }
    dim3 rgrid(total_q_rows, num_q_heads);
    if (head_dim == 64) hipLaunchKernelGGL((attn_reduce<64>), rgrid, dim3(64), 0, st, P);
    else hipLaunchKernelGGL((attn_reduce<128>), rgrid, dim3(64), 0, st, P);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        PKV_FAIL(KV_EDEVICE, "paged_attention_forward: launch failed: %s", hipGetErrorString(e));
    return KV_OK;
}

int kv_append_scatter(const void *k_new, const void *v_new, const int32_t *slot_mapping, int32_t n,
                      void *k_pool, void *v_pool, int32_t num_blocks, int32_t num_kv_heads,
                      int32_t head_dim, int32_t block_size, int32_t dtype, void *hip_stream) {
    using namespace pkv;
    if (dtype != KV_BF16 && dtype != KV_F32)
        PKV_FAIL(KV_EUNSUPPORTED, "kv_append_scatter: dtype %d not supported", dtype);
    if (block_size != kBlock)
        PKV_FAIL(KV_EUNSUPPORTED, "kv_append_scatter: block_size %d not supported (16)", block_size);
    if (head_dim <= 0 || head_dim % 16 || head_dim > 256)
        PKV_FAIL(KV_EUNSUPPORTED, "kv_append_scatter: head_dim %d not supported", head_dim);
    if (n < 0 || num_blocks < 0 || num_kv_heads <= 0)
        PKV_FAIL(KV_EINVAL, "kv_append_scatter: invalid size");
    if (n == 0) return KV_OK;
    if (!k_new || !v_new || !slot_mapping || !k_pool || !v_pool)
        PKV_FAIL(KV_EINVAL, "kv_append_scatter: required pointer is NULL");
    if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_pool) || !aligned16(v_pool))
        PKV_FAIL(KV_EINVAL, "kv_append_scatter: K/V and pools must be 16-byte aligned");
    if ((int64_t)num_blocks * kBlock > INT32_MAX) PKV_FAIL(KV_EINVAL, "kv_append_scatter: pool too large");
    const int X = dtype == KV_BF16 ? 8 : 4;
    const int64_t threads = (int64_t)n * num_kv_heads * (head_dim / X);
    const int64_t blocks = (threads + 255) / 256;
    if (blocks > INT32_MAX) PKV_FAIL(KV_EINVAL, "kv_append_scatter: too many tokens");
    hipStream_t st = reinterpret_cast<hipStream_t>(hip_stream);
    (void)hipGetLastError();
    if (dtype == KV_BF16)
        hipLaunchKernelGGL(scatter_kernel<uint16_t>, dim3((unsigned)blocks), dim3(256), 0, st,
                           static_cast<const uint16_t *>(k_new), static_cast<const uint16_t *>(v_new), slot_mapping,
                           n, static_cast<uint16_t *>(k_pool), static_cast<uint16_t *>(v_pool), num_blocks,
                           num_kv_heads, head_dim);
    else
        hipLaunchKernelGGL(scatter_kernel<float>, dim3((unsigned)blocks), dim3(256), 0, st,
                           static_cast<const float *>(k_new), static_cast<const float *>(v_new), slot_mapping, n,
                           static_cast<float *>(k_pool), static_cast<float *>(v_pool), num_blocks, num_kv_heads,
                           head_dim);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) PKV_FAIL(KV_EDEVICE, "kv_append_scatter: launch failed: %s", hipGetErrorString(e));
    return KV_OK;
}

}  // extern "C"
