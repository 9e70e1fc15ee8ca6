// Batched attention over a paged KV cache, and the paged K/V scatter-write,
// for gfx950 (CDNA4, wave64).
//
// TensorSharp "高级功能" page, section "原生分页注意力": one native call gathers
// K/V through the paged buffers for many sequences and runs fused attention,
// with a variant taking per-head sink logits; its "批量前向" paragraph pairs the
// batched forward with a paged K/V scatter-write. Decode rows, chunked-prefill
// rows (section "性能优化", chunked prefill) and speculative-verify windows
// (section "MTP / NextN 推测解码") share one entry point. The TensorFold pages
// (sections on the exactness rule and on row-invariant wide-window kernels)
// require that a row computed alone and the same row inside a window give
// identical bits; every choice below that fixes an order of floating-point
// operations exists for that.
//
// Arithmetic of one (query row, query head), the same whatever batch, window,
// q_len or launch shape surrounds the row:
//  * absolute key positions are cut into splits (split_begin) and every split
//    into four quarters; a quarter's keys are consumed in 32-key chunks (two
//    16-token blocks) in ascending order by an online softmax in base 2;
//  * bf16: S^T = K Q^T and O^T = V^T P^T on 16x16x32 bf16 MFMA tiles, whose
//    per-element results do not depend on the row's position in the tile; P
//    enters the PV product as a hi + lo pair of bf16 values;
//  * the four quarter states fold left to right into a split state, the split
//    states fold left to right into the row state (fold_state), and the sink
//    and the one division come last (finalize), which writes +0 for every
//    zero output;
//  * fp32: one wave per (row, head), one online state over all keys in order.
// Two bf16 launch shapes compute exactly that: "parallel" (one workgroup per
// split, a wave per quarter, then a fold launch over the split states) for
// decode and verify rows, and "sequential" (one workgroup per 64 rows walking
// every split: quarter and split states in registers, the row state in LDS)
// for prefill chunks.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <mutex>
#include <type_traits>

#include "pagedkv.h"
#include "status.h"

namespace pkv {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

constexpr int kBlock = 16;
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kMaxHeadDim = 128;
constexpr int kParRows = 32;   // rows per (sequence, KV head) the parallel shape takes
constexpr int kSeqRows = 64;   // rows per workgroup in the sequential shape

// Tile formats of the MFMA paths: bf16 values, 8-bit codes, 4-bit codes.
constexpr int kKvBf16 = 0, kKvFp8 = 1, kKvFp4 = 2;

// ---------------------------------------------------------------------------
// Fixed partition of absolute key positions: 256-key splits below 1024,
// 1024-key splits from there on; each split has four equal quarters. (Short
// contexts get enough splits to spread over the CUs; long ones few partial
// states to fold.)
// ---------------------------------------------------------------------------
constexpr int kEdge = 1024, kSplitA = 256, kSplitB = 1024;
constexpr int kSplitsA = kEdge / kSplitA;
static_assert((kSplitA & (kSplitA - 1)) == 0 && (kSplitB & (kSplitB - 1)) == 0 && kEdge % kSplitB == 0,
              "split sizes are powers of two and the edge falls on a large-split boundary");

__host__ __device__ inline int split_index(int pos) {
    return pos < kEdge ? pos / kSplitA : kSplitsA + (pos - kEdge) / kSplitB;
}
__host__ __device__ inline int split_begin(int idx) {
    return idx < kSplitsA ? idx * kSplitA : kEdge + (idx - kSplitsA) * kSplitB;
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
    float2 *ws_ml;      // [rows][Hq][max_splits]: split max (log2 units), split sum
    float *ws_acc;      // [rows][Hq][max_splits][D]
    float *out;         // [rows][Hq][D]
    int32_t num_seqs, total_rows, Hq, Hkv, G, max_blocks_per_seq, num_blocks, max_splits;
    // split slots per sequence in the parallel grid: max_splits, or under a
    // sliding window the splits from the one holding the sequence's lowest
    // visible key on (no more can hold a visible key)
    int32_t grid_splits;
    int32_t decode_only;  // every sequence has q_len == 1 (rows packed in sequence order)
    // sequence slots per split slot in the parallel grid (>= num_seqs), or 0:
    // the grid is dealt in the balanced order of balanced_item
    int32_t seq_stride;
    float scale_log2;
    // Appending decode step (paged_attention_append_forward), else all null:
    // row s's own token sits at position ctx - 1; its K/V rows, and the pool
    // slot the split holding that position writes them to.
    const uint16_t *k_new, *v_new;
    const int32_t *slots;
    uint16_t *kp_w, *vp_w;
    // Shared prompt prefix (paged_attention_prefix_forward), else all 0:
    // sequences 0 .. pre_seqs - 1 are taken in groups of pre_m consecutive
    // sequences, and splits 0 .. pre_splits - 1 (wholly inside the prefix)
    // of a group are one item (see prefix_slot). pre_a: slots of the prefix
    // sequences' own splits (pre_seqs * (max_splits - pre_splits)).
    int32_t pre_seqs, pre_m, pre_groups, pre_splits, pre_a;
    // Restricted visibility (paged_attention_masked_forward), else null / 0:
    // one ancestor mask word per query row of a tree window, and a sliding
    // window of `window` keys ending at each row's position.
    const uint32_t *tree_mask;
    int32_t window;
};

// A zero (block, head) tile: loads of blocks past the end of a sequence read it.
__device__ __attribute__((aligned(16))) uint16_t g_zero_tile[kBlock * kMaxHeadDim];

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ inline float bcast(float v, int lane) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}

// ---------------------------------------------------------------------------
// Online-softmax state of one 16-row MFMA tile held by one wave. Lane 16g+n
// holds row n: its max m (log2 units), its sum l, and O^T[d][n] for
// d = 16 dt + 4 g + i in acc[dt][i].
// ---------------------------------------------------------------------------
template <int DT>
struct TileState {
    float m, l;
    f32x4_t acc[DT];
};

template <int DT>
__device__ inline void state_clear(TileState<DT> &s) {
    s.m = -INFINITY;
    s.l = 0.f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) s.acc[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
}

// a := a (+) b, the online-softmax merge of two states over disjoint keys.
// An empty state (m = -inf) is the identity, exactly.
template <int DT>
__device__ inline void fold_state(TileState<DT> &a, const TileState<DT> &b) {
    if (b.m == -INFINITY) return;
    if (a.m == -INFINITY) {
        a = b;
        return;
    }
    const float M = fmaxf(a.m, b.m);
    const float al = fast_exp2(a.m - M);
    const float be = fast_exp2(b.m - M);
    a.l = fmaf(a.l, al, b.l * be);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i) a.acc[dt][i] = fmaf(a.acc[dt][i], al, b.acc[dt][i] * be);
    a.m = M;
}

// fold_state without branches, for states whose empty members (m = -inf)
// may hold any finite l and accumulators rather than zeros: an empty b weighs
// 0 (be = 2^-inf) against a's weight 1, an empty a weighs 0 against b's 1,
// and otherwise the arithmetic is fold_state's, so every value equals
// fold_state's over cleared states (the sign of a zero aside, which finalize
// removes). Both empty: a stays empty. Lets a shape that folds often skip
// clearing the accumulators it has just folded.
// (fmaf(x, y, z) with the result in x's register: the compiler's own
// choice, z's register plus a copy back, costs 16 64-bit moves per fold.)
__device__ inline float fma_in_place(float x, float y, float z) {
    asm("v_fma_f32 %0, %0, %1, %2" : "+v"(x) : "v"(y), "v"(z));
    return x;
}

template <int DT>
__device__ inline void fold_state_flat(TileState<DT> &a, const TileState<DT> &b) {
    const float M = fmaxf(a.m, b.m);
    const float Mu = M == -INFINITY ? 0.f : M;
    const float al = b.m == -INFINITY ? 1.f : fast_exp2(a.m - Mu);
    const float be = fast_exp2(b.m - Mu);
    a.l = fmaf(a.l, al, b.l * be);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i) a.acc[dt][i] = fma_in_place(a.acc[dt][i], al, b.acc[dt][i] * be);
    a.m = M;
}

// out = acc / (l + sink term); the sink logit (log2 units, -inf if none)
// takes part in the max. A zero output is written as +0 (x + 0 turns -0 into
// +0 and keeps every other value): a row's accumulators carry its values
// exactly through steps in which it sees no key, but not always the sign of
// a zero (see step_core).
template <int DT>
__device__ inline void finalize(const TileState<DT> &s, float sink2, f32x4_t *o) {
    float l = s.l;
    float al = 1.f;
    if (sink2 != -INFINITY) {
        const float M = fmaxf(s.m, sink2);
        al = fast_exp2(s.m - M);
        l = fmaf(l, al, fast_exp2(sink2 - M));
    }
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i) o[dt][i] = (s.acc[dt][i] * al) / l + 0.0f;
}

// ---------------------------------------------------------------------------
// One online-softmax step: a 32-key chunk, blocks b0 and b1. Lane 16g+n.
// Key slots: the S^T tile tau row m holds token 8((m/4)%2) + 4tau + m%4 of
// block m/8, so that after the QK product lane 16g+n holds, for its row n,
// the scores of tokens 8(g%2)..8(g%2)+7 of block g/2 (tile 0 the first four,
// tile 1 the last four). Those eight keys are the lane's k-slots of the PV
// product, whose V^T operand is then one 16-byte run of the V block.
//   k[tau][j]: K of key slot (tau, n), channels 32j+8g..+7
//   v[dt]:     V^T of channel 16dt+n at the lane's eight keys
//   qop[j]:    Q of row n, channels 32j+8g..+7
// Key kc + key_off(g) + 4tau + i is visible to the lane's row when <= prow.
// ---------------------------------------------------------------------------
constexpr int kStep = 32;
__device__ inline int key_off(int g) { return 16 * (g >> 1) + 8 * (g & 1); }

template <int D>
struct StepRegs {
    u32x4_t k[2][D / 32];
    u32x4_t v[D / 16];
};

// K/V operands of one chunk; kb0/vb0 and kb1/vb1 point at the K and V tiles
// of its two blocks (global memory or LDS).
template <int D>
__device__ inline void load_step(StepRegs<D> &r, const uint16_t *kb0, const uint16_t *vb0, const uint16_t *kb1,
                                 const uint16_t *vb1, int g, int n) {
    const uint16_t *k = n >= 8 ? kb1 : kb0;
    const int tk = 8 * ((n >> 2) & 1) + (n & 3);  // token of key slot n, tile 0
#pragma unroll
    for (int j = 0; j < D / 32; ++j) {
        r.k[0][j] = *reinterpret_cast<const u32x4_t *>(k + ((4 * j + g) * kBlock + tk) * 8);
        r.k[1][j] = *reinterpret_cast<const u32x4_t *>(k + ((4 * j + g) * kBlock + tk + 4) * 8);
    }
    const uint16_t *v = (g >> 1) ? vb1 : vb0;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt)
        r.v[dt] = *reinterpret_cast<const u32x4_t *>(v + (16 * dt + n) * kBlock + 8 * (g & 1));
}

// The same operands from a step staged in LDS by attn_sequential, whose
// layout permutes 16-byte pieces so that the lanes of one LDS cycle read
// distinct banks, whether a cycle serves 8 lanes (128 bytes) or 16 (256):
// in a K tile the 16 tokens of a channel chunk sit in the order 0-3, 8-11,
// 4-7, 12-15 (lds_k_pos), the K tiles of the two blocks start 128 bytes
// apart modulo 256, and in a V tile the two 16-byte halves of channel row r
// swap when bit 2 xor bit 3 of r is set (lds_v_half). K tiles of blocks 0, 1
// at k0, k1; V tiles at v0, v1.
__device__ inline int lds_k_pos(int token) { return (token & 3) + ((token >> 3) << 2) + (((token >> 2) & 1) << 3); }
__device__ inline int lds_v_half(int row, int half) { return half ^ ((row >> 2) & 1) ^ ((row >> 3) & 1); }

template <int D>
__device__ inline void load_step_lds(StepRegs<D> &r, const uint16_t *k0, const uint16_t *v0, const uint16_t *k1,
                                     const uint16_t *v1, int g, int n) {
    const uint16_t *k = n >= 8 ? k1 : k0;
    const int pk = n & 7;  // lds_k_pos of the lane's tile-0 token; tile 1's follow 8 later
#pragma unroll
    for (int j = 0; j < D / 32; ++j) {
        r.k[0][j] = *reinterpret_cast<const u32x4_t *>(k + ((4 * j + g) * kBlock + pk) * 8);
        r.k[1][j] = *reinterpret_cast<const u32x4_t *>(k + ((4 * j + g) * kBlock + pk + 8) * 8);
    }
    const uint16_t *v = (g >> 1) ? v1 : v0;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
        const int row = 16 * dt + n;
        r.v[dt] = *reinterpret_cast<const u32x4_t *>(v + row * kBlock + 8 * lds_v_half(row, g & 1));
    }
}

// Zero V of keys at or past ctx, so that a zero weight never meets a NaN.
template <int D>
__device__ inline void mask_tail(StepRegs<D> &r, int kc, int ctx, int g) {
    if (kc + kStep <= ctx) return;
    const int nv = ctx - (kc + key_off(g));  // the lane's keys 0 .. nv-1 exist
    uint32_t m[4];
#pragma unroll
    for (int w = 0; w < 4; ++w) m[w] = (2 * w < nv ? 0x0000FFFFu : 0u) | (2 * w + 1 < nv ? 0xFFFF0000u : 0u);
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
        r.v[dt].x &= m[0];
        r.v[dt].y &= m[1];
        r.v[dt].z &= m[2];
        r.v[dt].w &= m[3];
    }
}

// Put the new token's K/V (held in registers: knew[j] = channels
// 32j+8g..+7, vnew[dt] = channel 16dt+n) into the operands of the step at kc
// that holds its position pn, in place of what the pool held there. Only
// fixed register indices and per-lane selects: a register array indexed by a
// run-time value would live in scratch memory.
template <int D>
__device__ inline void patch_new_key(StepRegs<D> &r, const u32x4_t (&knew)[D / 32], const uint32_t (&vnew)[D / 16],
                                     int kc, int pn, int g, int n) {
    const int hb = (pn - kc) >> 4, t = pn & (kBlock - 1);
    const int tk = 8 * ((n >> 2) & 1) + (n & 3);
    const bool kblk = (n >= 8) == (hb == 1);
    const bool k0 = kblk && tk == t, k1 = kblk && tk + 4 == t;
#pragma unroll
    for (int j = 0; j < D / 32; ++j) {
        r.k[0][j] = k0 ? knew[j] : r.k[0][j];
        r.k[1][j] = k1 ? knew[j] : r.k[1][j];
    }
    // V^T: the lane's eight keys are tokens 8(g&1)..+7 of block g>>1; the new
    // key is element e of them, the low or high half of 32-bit word e / 2
    const bool vm = (g >> 1) == hb && (t >> 3) == (g & 1);
    const int e = t & 7;
    const bool w0 = vm && (e >> 1) == 0, w1 = vm && (e >> 1) == 1, w2 = vm && (e >> 1) == 2, w3 = vm && (e >> 1) == 3;
    const uint32_t keep = (e & 1) ? 0x0000FFFFu : 0xFFFF0000u;
    const int sh = (e & 1) ? 16 : 0;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
        const uint32_t ins = vnew[dt] << sh;
        r.v[dt].x = w0 ? ((r.v[dt].x & keep) | ins) : r.v[dt].x;
        r.v[dt].y = w1 ? ((r.v[dt].y & keep) | ins) : r.v[dt].y;
        r.v[dt].z = w2 ? ((r.v[dt].z & keep) | ins) : r.v[dt].z;
        r.v[dt].w = w3 ? ((r.v[dt].w & keep) | ins) : r.v[dt].w;
    }
}

// P as bf16 hi + lo pairs: hi = w rounded to bf16 (nearest even), lo = the
// rest rounded to bf16; two values per conversion instruction.
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ inline void split_hi_lo(const float (&w)[8], bf16x8_t &phi, bf16x8_t &plo) {
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
        const auto h = __builtin_convertvector(f32x2_t{w[e], w[e + 1]}, bf16x2_t);
        const uint32_t hb = __builtin_bit_cast(uint32_t, h);
        const float h0 = __builtin_bit_cast(float, hb << 16), h1 = __builtin_bit_cast(float, hb & 0xFFFF0000u);
        const auto l = __builtin_convertvector(f32x2_t{w[e] - h0, w[e + 1] - h1}, bf16x2_t);
        phi[e] = h[0];
        phi[e + 1] = h[1];
        plo[e] = l[0];
        plo[e + 1] = l[1];
    }
}

// Reductions over the four lanes n, n + 16, n + 32, n + 48 that hold one
// row. The gfx950 lane swaps exchange rows 0/1 and 2/3 (16) or the two
// halves (32) of two copies of x, after which every lane holds the lower and
// the upper value of its pair: no trip through LDS. max and + are
// commutative, so both lanes of a pair get the same bits, the bits a
// lane-own + partner order gives.
__device__ inline float2 lane_pair16(float x) {
    const int v = __builtin_bit_cast(int, x);
    const auto s = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return make_float2(__builtin_bit_cast(float, (int)s[0]), __builtin_bit_cast(float, (int)s[1]));
}
__device__ inline float2 lane_pair32(float x) {
    const int v = __builtin_bit_cast(int, x);
    const auto s = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return make_float2(__builtin_bit_cast(float, (int)s[0]), __builtin_bit_cast(float, (int)s[1]));
}
__device__ inline float row_max4(float x) {
    float2 p = lane_pair16(x);
    p = lane_pair32(fmaxf(p.x, p.y));
    return fmaxf(p.x, p.y);
}
__device__ inline float row_sum4(float x) {
    float2 p = lane_pair16(x);
    p = lane_pair32(p.x + p.y);
    return p.x + p.y;
}

// One online-softmax step over the MFMA operands kop(tau, j) (K, tile tau,
// k-step j) and vop(dt) (V^T, d-tile dt). SCALED: 8-bit pools, whose scores
// take the keys' K scales (ksc, the lane's 8 keys) and whose probabilities
// take the keys' V scales (vsc) before the PV product; the sum l takes the
// unscaled probabilities.
// The keys one query row sees: positions up to prow; with a restricted
// visibility also none below lo, and of the tree window starting at wbase only
// those whose bit in tm is set (the row's own bit included). Unrestricted rows
// carry lo far below 0 and wbase far above any position.
struct RowVis {
    int prow;
    int lo;
    int wbase;
    uint32_t tm;
};

constexpr int kFarBelow = -(1 << 30), kFarAbove = 1 << 30;

// Visibility of the lane's 8 keys key0 .. key0 + 7 as bits 0 .. 7.
__device__ inline uint32_t visible8(const RowVis &v, int key0) {
    const int hi = v.prow - key0;  // keys i <= hi
    const int lo = v.lo - key0;    // keys i >= lo
    uint32_t m = hi >= 7 ? 0xFFu : hi < 0 ? 0u : (0xFFu >> (7 - hi));
    m &= lo <= 0 ? 0xFFu : lo >= 8 ? 0u : ((0xFFu << lo) & 0xFFu);
    // 64-bit word: bits 0..31 stand for the 32 keys below wbase (visible),
    // bits 32 + j for window key j
    const int sh = key0 - v.wbase + 32;
    const uint64_t ext = ((uint64_t)v.tm << 32) | 0xFFFFFFFFull;
    m &= sh < 0 ? 0xFFu : sh >= 64 ? 0u : (uint32_t)(ext >> sh) & 0xFFu;
    return m;
}

template <int D, bool SCALED, bool MASKED, bool ALWAYS = false, class KOp, class VOp>
__device__ inline void step_core(TileState<D / 16> &st, KOp kop, VOp vop, const float (&ksc)[8],
                                 const float (&vsc)[8], const u32x4_t (&qop)[D / 32], int kc, const RowVis &rv,
                                 int g, float scale_log2, bool fresh = false) {
    const int prow = rv.prow;
    constexpr int KJ = D / 32, DT = D / 16;
    f32x4_t s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < KJ; ++j) {
        const bf16x8_t b = __builtin_bit_cast(bf16x8_t, qop[j]);
        s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop(0, j), b, s0, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop(1, j), b, s1, 0, 0, 0);
    }
    float sc[8];
    const int lim = prow - (kc + key_off(g));  // the row sees the lane's keys 0 .. lim
    uint32_t vm = 0;
    if constexpr (MASKED) vm = visible8(rv, kc + key_off(g));
    auto vis = [&](int i) { return MASKED ? ((vm >> i) & 1u) != 0 : i <= lim; };
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if constexpr (SCALED) {
            sc[i] = (s0[i] * ksc[i]) * scale_log2;
            sc[4 + i] = (s1[i] * ksc[4 + i]) * scale_log2;
        } else {
            sc[i] = s0[i] * scale_log2;
            sc[4 + i] = s1[i] * scale_log2;
        }
    }
    // Masking only in steps where some lane does not see all its keys (the
    // diagonal, the tail, a window or tree edge); elsewhere it changes nothing.
    if (!__all(MASKED ? vm == 0xFFu : lim >= 7)) {
#pragma unroll
        for (int i = 0; i < 8; ++i) sc[i] = vis(i) ? sc[i] : -INFINITY;
    }
    const float mx =
        row_max4(fmaxf(fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3])), fmaxf(fmaxf(sc[4], sc[5]), fmaxf(sc[6], sc[7]))));
    // the row sees at least one key of the chunk (with a restricted
    // visibility: its maximum over the chunk is a score)
    const bool has = MASKED ? mx != -INFINITY : kc <= prow;
    const float m_new = fmaxf(st.m, mx);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = fast_exp2(st.m - m_use);
    float pv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) pv[e] = fast_exp2(sc[e] - m_use);
    const float rs = row_sum4(((pv[0] + pv[1]) + (pv[2] + pv[3])) + ((pv[4] + pv[5]) + (pv[6] + pv[7])));
    bf16x8_t phi, plo;
    {
        float w[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) w[e] = SCALED ? pv[e] * vsc[e] : pv[e];
        split_hi_lo(w, phi, plo);
    }
    // A row with no visible key in the chunk keeps m and l (selects), and
    // its accumulators keep their values: alpha is 1 (x * 1 == x, denormals
    // are kept) or the accumulators are still zero, and its weights are 0
    // against finite V (masked tails are zeroed), so the products add zeros.
    // Only a zero's sign can change (-0 + 0 = +0), which finalize removes.
    // ALWAYS (the prefill shape, where some row's max moves in most steps):
    // the rescale runs unconditionally, the same values (x * 1 == x), so that
    // the accumulators keep one set of registers through the step.
    // fresh (ALWAYS only, uniform): the first step of a quarter whose state
    // was emptied by its max alone; every row's alpha is 0, so the
    // accumulators restart from zero in the MFMA instead of being scaled by 0
    // (the same values; only a zero's sign could differ).
    if (ALWAYS && fresh) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            const bf16x8_t va = vop(dt);
            st.acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, plo, f32x4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
            st.acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, phi, st.acc[dt], 0, 0, 0);
        }
    } else {
        if (ALWAYS || __any(alpha != 1.f)) {
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) st.acc[dt] *= alpha;
        }
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            const bf16x8_t va = vop(dt);
            st.acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, plo, st.acc[dt], 0, 0, 0);
            st.acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, phi, st.acc[dt], 0, 0, 0);
        }
    }
    const float l_new = fmaf(alpha, st.l, rs);
    st.l = has ? l_new : st.l;
    st.m = has ? m_new : st.m;
}

// Two 16-row tiles through one step: each K operand piece meets both tiles'
// score MFMAs and each V operand piece both tiles' PV MFMAs as soon as it is
// formed, so no converted operand outlives its use. Per tile the sequence of
// operations is step_core's exactly.
template <int D, bool SCALED, bool MASKED, class KOp, class VOp>
__device__ inline void step_core2(TileState<D / 16> (&st)[2], KOp kop, VOp vop, const float (&ksc)[8],
                                  const float (&vsc)[8], const u32x4_t (&qop)[2][D / 32], int kc,
                                  const RowVis (&rv)[2], int g, float scale_log2) {
    constexpr int KJ = D / 32, DT = D / 16;
    f32x4_t s0[2], s1[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) s0[t] = s1[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < KJ; ++j) {
        const bf16x8_t k0 = kop(0, j), k1 = kop(1, j);
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const bf16x8_t b = __builtin_bit_cast(bf16x8_t, qop[t][j]);
            s0[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0, b, s0[t], 0, 0, 0);
            s1[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1, b, s1[t], 0, 0, 0);
        }
    }
    bf16x8_t phi[2], plo[2];
    float alpha[2], m_new[2], rs[2];
    bool has[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const int prow = rv[t].prow;
        float sc[8];
        const int lim = prow - (kc + key_off(g));
        uint32_t vm = 0;
        if constexpr (MASKED) vm = visible8(rv[t], kc + key_off(g));
        auto vis = [&](int i) { return MASKED ? ((vm >> i) & 1u) != 0 : i <= lim; };
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if constexpr (SCALED) {
                sc[i] = (s0[t][i] * ksc[i]) * scale_log2;
                sc[4 + i] = (s1[t][i] * ksc[4 + i]) * scale_log2;
            } else {
                sc[i] = s0[t][i] * scale_log2;
                sc[4 + i] = s1[t][i] * scale_log2;
            }
        }
        if (!__all(MASKED ? vm == 0xFFu : lim >= 7)) {  // as in step_core
#pragma unroll
            for (int i = 0; i < 8; ++i) sc[i] = vis(i) ? sc[i] : -INFINITY;
        }
        const float mx = row_max4(
            fmaxf(fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3])), fmaxf(fmaxf(sc[4], sc[5]), fmaxf(sc[6], sc[7]))));
        has[t] = MASKED ? mx != -INFINITY : kc <= prow;
        m_new[t] = fmaxf(st[t].m, mx);
        const float m_use = m_new[t] == -INFINITY ? 0.f : m_new[t];
        alpha[t] = fast_exp2(st[t].m - m_use);
        float pv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) pv[e] = fast_exp2(sc[e] - m_use);
        rs[t] = row_sum4(((pv[0] + pv[1]) + (pv[2] + pv[3])) + ((pv[4] + pv[5]) + (pv[6] + pv[7])));
        float w[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) w[e] = SCALED ? pv[e] * vsc[e] : pv[e];
        split_hi_lo(w, phi[t], plo[t]);
    }
    // as in step_core, for both tiles at once
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        if (__any(alpha[t] != 1.f)) {
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) st[t].acc[dt] *= alpha[t];
        }
    }
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
        const bf16x8_t va = vop(dt);
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            st[t].acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, plo[t], st[t].acc[dt], 0, 0, 0);
            st[t].acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, phi[t], st[t].acc[dt], 0, 0, 0);
        }
    }
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const float l_new = fmaf(alpha[t], st[t].l, rs[t]);
        st[t].l = has[t] ? l_new : st[t].l;
        st[t].m = has[t] ? m_new[t] : st[t].m;
    }
}

template <int D, bool MASKED, bool ALWAYS = false>
__device__ inline void step_update(TileState<D / 16> &st, const StepRegs<D> &r, const u32x4_t (&qop)[D / 32], int kc,
                                   const RowVis &rv, int g, float scale_log2, bool fresh = false) {
    const float none[8] = {};
    step_core<D, false, MASKED, ALWAYS>(
        st, [&](int tau, int j) { return __builtin_bit_cast(bf16x8_t, r.k[tau][j]); },
        [&](int dt) { return __builtin_bit_cast(bf16x8_t, r.v[dt]); }, none, none, qop, kc, rv, g, scale_log2, fresh);
}

template <int D, bool MASKED>
__device__ inline void step_update2(TileState<D / 16> (&st)[2], const StepRegs<D> &r, const u32x4_t (&qop)[2][D / 32],
                                    int kc, const RowVis (&rv)[2], int g, float scale_log2) {
    const float none[8] = {};
    step_core2<D, false, MASKED>(
        st, [&](int tau, int j) { return __builtin_bit_cast(bf16x8_t, r.k[tau][j]); },
        [&](int dt) { return __builtin_bit_cast(bf16x8_t, r.v[dt]); }, none, none, qop, kc, rv, g, scale_log2);
}

// ---------------------------------------------------------------------------
// 8-bit pools: FP8 E4M3 codes (OCP E4M3FN) with one float32 scale per
// (token, KV head); the stored value is code * scale. Tile of a (block, KV
// head): 16 * D code bytes, then the 16 tokens' scales. Within the codes
//   K: token t, channel c = 64 p + 32 jj + 8 g + e  at byte ((p*4 + g)*16 + t)*16 + jj*8 + e
//   V: token t = 8 h + e, channel c = 16 (2 d + dd) + n  at byte (((d*16 + n)*2 + h)*2 + dd)*8 + e
// so that one 16-byte load gives a lane its K operands of two MFMA k-steps,
// or its V^T operands of two d-tiles. Codes become bf16 exactly; scales act
// in float32 on the scores (K) and on the probabilities (V).
// ---------------------------------------------------------------------------

template <int D>
constexpr int q8_tile_bytes() { return 16 * D + 64; }

template <int D>
struct StepRegs8 {
    u32x4_t k[2][D / 64];  // tile tau, channel pair p
    u32x4_t v[D / 32];     // d-tile pair
    f32x4_t ks[2], vs[2];  // scales of the lane's keys 0-3 and 4-7
};

// eight codes (two dwords, low byte first) -> eight bf16 values, exact
__device__ inline bf16x8_t fp8x8_to_bf16(uint32_t lo, uint32_t hi) {
    const bf16x2_t a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
    const bf16x2_t b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
    const bf16x2_t c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
    const bf16x2_t d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
    return bf16x8_t{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// Operands of one chunk from 8-bit tiles kt0/vt0 and kt1/vt1 (blocks 0, 1).
// kpos(t): position of token t's K pieces, vhalf(row, h): position of V half
// h of channel row `row` (identity in the pools; swizzled in LDS staging).
template <int D, class KPos, class VHalf>
__device__ inline void load_step8(StepRegs8<D> &r, const uint8_t *kt0, const uint8_t *vt0, const uint8_t *kt1,
                                  const uint8_t *vt1, int g, int n, KPos kpos, VHalf vhalf) {
    const uint8_t *k = n >= 8 ? kt1 : kt0;
    const int tk = 8 * ((n >> 2) & 1) + (n & 3);
#pragma unroll
    for (int p = 0; p < D / 64; ++p) {
        r.k[0][p] = *reinterpret_cast<const u32x4_t *>(k + ((p * 4 + g) * kBlock + kpos(tk)) * 16);
        r.k[1][p] = *reinterpret_cast<const u32x4_t *>(k + ((p * 4 + g) * kBlock + kpos(tk + 4)) * 16);
    }
    const uint8_t *v = (g >> 1) ? vt1 : vt0;
#pragma unroll
    for (int d = 0; d < D / 32; ++d)
        r.v[d] = *reinterpret_cast<const u32x4_t *>(v + ((d * 16 + n) * 2 + vhalf(d * 16 + n, g & 1)) * 16);
    const uint8_t *kss = ((g >> 1) ? kt1 : kt0) + 16 * D + 32 * (g & 1);
    const uint8_t *vss = v + 16 * D + 32 * (g & 1);
    r.ks[0] = *reinterpret_cast<const f32x4_t *>(kss);
    r.ks[1] = *reinterpret_cast<const f32x4_t *>(kss + 16);
    r.vs[0] = *reinterpret_cast<const f32x4_t *>(vss);
    r.vs[1] = *reinterpret_cast<const f32x4_t *>(vss + 16);
}

template <int D>
__device__ inline void load_step8(StepRegs8<D> &r, const uint8_t *kt0, const uint8_t *vt0, const uint8_t *kt1,
                                  const uint8_t *vt1, int g, int n) {
    load_step8<D>(r, kt0, vt0, kt1, vt1, g, n, [](int t) { return t; }, [](int, int h) { return h; });
}

// Zero V codes and V scales of keys at or past ctx, so that a zero weight
// never meets a NaN (the scores of those keys are masked by select).
template <int D>
__device__ inline void mask_tail8(StepRegs8<D> &r, int kc, int ctx, int g) {
    if (kc + kStep <= ctx) return;
    const int nv = ctx - (kc + key_off(g));  // the lane's keys 0 .. nv-1 exist
    auto bytes = [](int k) {                 // low k bytes of a dword set, 0 <= k <= 4
        return k <= 0 ? 0u : k >= 4 ? 0xFFFFFFFFu : (1u << (8 * k)) - 1u;
    };
    const uint32_t m0 = bytes(nv), m1 = bytes(nv - 4);
#pragma unroll
    for (int d = 0; d < D / 32; ++d) {
        r.v[d].x &= m0;
        r.v[d].y &= m1;
        r.v[d].z &= m0;
        r.v[d].w &= m1;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        r.vs[0][i] = i < nv ? r.vs[0][i] : 0.f;
        r.vs[1][i] = i + 4 < nv ? r.vs[1][i] : 0.f;
    }
}

// The K and V scales of the lane's eight keys (8- and 4-bit operands).
template <class R>
__device__ inline void step_scales(const R &r, float (&ksc)[8], float (&vsc)[8]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        ksc[i] = r.ks[0][i];
        ksc[4 + i] = r.ks[1][i];
        vsc[i] = r.vs[0][i];
        vsc[4 + i] = r.vs[1][i];
    }
}

template <int D, bool MASKED>
__device__ inline void step_update8x2(TileState<D / 16> (&st)[2], const StepRegs8<D> &r,
                                      const u32x4_t (&qop)[2][D / 32], int kc, const RowVis (&rv)[2], int g,
                                      float scale_log2) {
    float ksc[8], vsc[8];
    step_scales(r, ksc, vsc);
    step_core2<D, true, MASKED>(
        st,
        [&](int tau, int j) {
            const u32x4_t w = r.k[tau][j >> 1];
            return (j & 1) ? fp8x8_to_bf16(w.z, w.w) : fp8x8_to_bf16(w.x, w.y);
        },
        [&](int dt) {
            const u32x4_t w = r.v[dt >> 1];
            return (dt & 1) ? fp8x8_to_bf16(w.z, w.w) : fp8x8_to_bf16(w.x, w.y);
        },
        ksc, vsc, qop, kc, rv, g, scale_log2);
}

template <int D, bool MASKED, bool ALWAYS = false>
__device__ inline void step_update8(TileState<D / 16> &st, const StepRegs8<D> &r, const u32x4_t (&qop)[D / 32],
                                    int kc, const RowVis &rv, int g, float scale_log2, bool fresh = false) {
    float ksc[8], vsc[8];
    step_scales(r, ksc, vsc);
    step_core<D, true, MASKED, ALWAYS>(
        st,
        [&](int tau, int j) {
            const u32x4_t w = r.k[tau][j >> 1];
            return (j & 1) ? fp8x8_to_bf16(w.z, w.w) : fp8x8_to_bf16(w.x, w.y);
        },
        [&](int dt) {
            const u32x4_t w = r.v[dt >> 1];
            return (dt & 1) ? fp8x8_to_bf16(w.z, w.w) : fp8x8_to_bf16(w.x, w.y);
        },
        ksc, vsc, qop, kc, rv, g, scale_log2, fresh);
}

// Pool access of the parallel and sequential shapes for each tile format
// (kKvBf16, kKvFp8, kKvFp4); pointers are byte addresses of tiles.
template <int D, int KF>
struct Pool;

template <int D>
struct Pool<D, kKvBf16> {
    using Regs = StepRegs<D>;
    static constexpr size_t tile_bytes = (size_t)kBlock * D * 2;
    __device__ static void load(Regs &r, const uint8_t *k0, const uint8_t *v0, const uint8_t *k1, const uint8_t *v1,
                                int g, int n) {
        load_step<D>(r, reinterpret_cast<const uint16_t *>(k0), reinterpret_cast<const uint16_t *>(v0),
                     reinterpret_cast<const uint16_t *>(k1), reinterpret_cast<const uint16_t *>(v1), g, n);
    }
    __device__ static void mask(Regs &r, int kc, int ctx, int g) { mask_tail<D>(r, kc, ctx, g); }
    template <bool MASKED, bool ALWAYS = false>
    __device__ static void update(TileState<D / 16> &st, const Regs &r, const u32x4_t (&qop)[D / 32], int kc,
                                  const RowVis &rv, int g, float sl2, bool fresh = false) {
        step_update<D, MASKED, ALWAYS>(st, r, qop, kc, rv, g, sl2, fresh);
    }
    template <bool MASKED>
    __device__ static void update2(TileState<D / 16> (&st)[2], const Regs &r, const u32x4_t (&qop)[2][D / 32], int kc,
                                   const RowVis (&rv)[2], int g, float sl2) {
        step_update2<D, MASKED>(st, r, qop, kc, rv, g, sl2);
    }
};

template <int D>
struct Pool<D, kKvFp8> {
    using Regs = StepRegs8<D>;
    static constexpr size_t tile_bytes = (size_t)q8_tile_bytes<D>();
    __device__ static void load(Regs &r, const uint8_t *k0, const uint8_t *v0, const uint8_t *k1, const uint8_t *v1,
                                int g, int n) {
        load_step8<D>(r, k0, v0, k1, v1, g, n);
    }
    __device__ static void mask(Regs &r, int kc, int ctx, int g) { mask_tail8<D>(r, kc, ctx, g); }
    template <bool MASKED, bool ALWAYS = false>
    __device__ static void update(TileState<D / 16> &st, const Regs &r, const u32x4_t (&qop)[D / 32], int kc,
                                  const RowVis &rv, int g, float sl2, bool fresh = false) {
        step_update8<D, MASKED, ALWAYS>(st, r, qop, kc, rv, g, sl2, fresh);
    }
    template <bool MASKED>
    __device__ static void update2(TileState<D / 16> (&st)[2], const Regs &r, const u32x4_t (&qop)[2][D / 32], int kc,
                                   const RowVis (&rv)[2], int g, float sl2) {
        step_update8x2<D, MASKED>(st, r, qop, kc, rv, g, sl2);
    }
};

// ---------------------------------------------------------------------------
// 4-bit pools: FP4 E2M1 codes (OCP) with one float32 scale per (token, KV
// head); the stored value is code * scale. Tile of a (block, KV head): 8 * D
// code bytes, two codes a byte (the first in the low nibble), then the 16
// tokens' scales. Code (nibble) index of token t, channel c:
//   K: c = 32 j + 8 g + e  at  ((g*16 + t) * (D/32) + j) * 8 + e
//   V: t = 8 h + e, c = 16 dt + n  at  ((n*2 + h) * (D/16) + dt) * 8 + e
// so that a lane's K operands for a key are one run of D/8 bytes (a dword
// per MFMA k-step) and its V^T operands one run of D/4 bytes (a dword per
// d-tile). Two keys share each V byte, which is why a token written alone
// takes atomic nibble updates (scatter4_kernel).
// ---------------------------------------------------------------------------
template <int D>
constexpr int q4_tile_bytes() { return 8 * D + 64; }

template <int D>
struct StepRegs4 {
    uint32_t k[2][D / 32];  // tile tau: dword j = channels 32j+8g..+7 of the lane's key
    uint32_t v[D / 16];     // dword dt = channel 16dt+n at the lane's eight keys
    f32x4_t ks[2], vs[2];   // scales of the lane's keys 0-3 and 4-7
};

// eight codes (one dword, low nibble first) -> eight bf16 values, exact
__device__ inline bf16x8_t fp4x8_to_bf16(uint32_t w) {
    const bf16x2_t a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 0);
    const bf16x2_t b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 1);
    const bf16x2_t c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 2);
    const bf16x2_t d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 3);
    return bf16x8_t{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

__device__ inline void load_dw2(uint32_t *d, const uint8_t *src) {
    const u32x2_t w = *reinterpret_cast<const u32x2_t *>(src);
    d[0] = w.x;
    d[1] = w.y;
}
__device__ inline void load_dw4(uint32_t *d, const uint8_t *src) {
    const u32x4_t w = *reinterpret_cast<const u32x4_t *>(src);
    d[0] = w.x;
    d[1] = w.y;
    d[2] = w.z;
    d[3] = w.w;
}

// Asynchronous copy of 16 bytes per lane from global memory (sbase + voff)
// to LDS (lds + 16 * lane): the gfx950 global-to-LDS load, counted by vmcnt.
// sbase and lds must be wave-uniform; both are read from the first lane into
// scalar registers. It has no register result; the compiler does not see
// the LDS write, so the caller waits for vmcnt and synchronises the
// workgroup before any wave reads the bytes, and waits again before the
// workgroup ends. M0 carries the LDS address and is restored afterwards.
__device__ inline void lds_copy16(const void *sbase, uint32_t voff, uint32_t lds) {
    // (readfirstlane returns int: each half goes through uint32_t before it
    // widens, or a low half with bit 31 set would fill the high half with ones)
    const uint64_t a = (uint64_t)(uintptr_t)sbase;
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a);
    const uint64_t u = ((uint64_t)hi << 32) | lo;
    const uint32_t l = (uint32_t)__builtin_amdgcn_readfirstlane((int)lds);
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %3\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, %2\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(voff), "s"((const void *)(uintptr_t)u), "s"(l)
        : "memory");
}
__device__ inline uint32_t lds_addr(const void *p) {
    return (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p);
}
// A wave-uniform load through the scalar cache (read-only data).
__device__ inline int32_t load_scalar(const int32_t *p) { return *(const __attribute__((address_space(4))) int32_t *)p; }

// Staged copies in LDS (attn_sequential) permute 16-byte pieces so that the
// 8 or 16 lanes of one LDS cycle read distinct banks: at D = 128 a K piece is
// one token's run, kept in lds_k_pos order; a V piece c of channel row m's
// run (piece 4m + c, c = 2h + q, at D = 128; 2m + h at D = 64) moves within
// the row to c ^ f(m), f(m) = 2 b2 + (b1 ^ b3) at D = 128 and b2 ^ b3 at
// D = 64 (b_i = bit i of m). For every 8 consecutive rows, and for every 16,
// each piece column then lands in distinct 16-byte bank groups.
template <int D>
__device__ inline int lds_v4_piece(int pc) {
    if constexpr (D == 128)
        return (pc & ~3) | ((pc & 3) ^ ((((pc >> 4) & 1) << 1) | (((pc >> 3) ^ (pc >> 5)) & 1)));
    else return (pc & ~1) | ((pc & 1) ^ (((pc >> 3) ^ (pc >> 4)) & 1));
}

// LDS copies of a tile (16-byte pieces, staged by global-to-LDS copies that
// write lane l's piece at position l): the piece that belongs at position i,
// for the layouts load_step_lds, load_step8 and load_step4 read. K keeps the
// token order 0-3, 8-11, 4-7, 12-15 within each 16-piece chunk; V pieces of
// a channel row are permuted by the row's bits; scales stay in place. Both
// permutations are their own inverses (the token order swaps bits 2 and 3
// of the token; the V permutations flip low bits of the piece index by its
// higher bits), so position and source piece may be read either way.
template <int D, int KF>
__device__ inline int lds_k_piece(int i) {
    if constexpr (KF == kKvFp4) {
        if (D != 128 || i >= D / 2) return i;  // 8-byte runs in order; scales
    } else if constexpr (KF == kKvFp8) {
        if (i >= D) return i;  // scales
    }
    return (i >> 4) * kBlock + lds_k_pos(i & 15);
}
template <int D, int KF>
__device__ inline int lds_v_piece(int i) {
    if constexpr (KF == kKvFp4) return i >= D / 2 ? i : lds_v4_piece<D>(i);
    else if constexpr (KF == kKvFp8) return i >= D ? i : (i >> 1) * 2 + lds_v_half(i >> 1, i & 1);
    else return (i >> 1) * 2 + lds_v_half(i >> 1, i & 1);
}


// Operands of one chunk from 4-bit tiles kt0/vt0 and kt1/vt1 (blocks 0, 1),
// in the pools (LDS = false) or staged in LDS.
template <int D, bool LDS>
__device__ inline void load_step4(StepRegs4<D> &r, const uint8_t *kt0, const uint8_t *vt0, const uint8_t *kt1,
                                  const uint8_t *vt1, int g, int n) {
    constexpr int KB = D / 8, VB = D / 4;  // bytes of a K run, of a V run
    const uint8_t *k = n >= 8 ? kt1 : kt0;
    const int tk = 8 * ((n >> 2) & 1) + (n & 3);
#pragma unroll
    for (int tau = 0; tau < 2; ++tau) {
        const int t = tk + 4 * tau;
        if constexpr (D == 128) load_dw4(r.k[tau], k + (g * kBlock + (LDS ? lds_k_pos(t) : t)) * KB);
        else load_dw2(r.k[tau], k + (g * kBlock + t) * KB);
    }
    const uint8_t *v = (g >> 1) ? vt1 : vt0;
    const int h = g & 1;
#pragma unroll
    for (int q = 0; q < VB / 16; ++q) {
        const int pc = (2 * n + h) * (VB / 16) + q;
        load_dw4(r.v + 4 * q, v + (LDS ? lds_v4_piece<D>(pc) : pc) * 16);
    }
    const uint8_t *kss = ((g >> 1) ? kt1 : kt0) + 8 * D + 32 * h;
    const uint8_t *vss = v + 8 * D + 32 * h;
    r.ks[0] = *reinterpret_cast<const f32x4_t *>(kss);
    r.ks[1] = *reinterpret_cast<const f32x4_t *>(kss + 16);
    r.vs[0] = *reinterpret_cast<const f32x4_t *>(vss);
    r.vs[1] = *reinterpret_cast<const f32x4_t *>(vss + 16);
}

// Zero the V scales of keys at or past ctx, so that a zero weight never meets
// a NaN (codes are always finite; the scores of those keys are masked by select).
template <int D>
__device__ inline void mask_tail4(StepRegs4<D> &r, int kc, int ctx, int g) {
    if (kc + kStep <= ctx) return;
    const int nv = ctx - (kc + key_off(g));  // the lane's keys 0 .. nv-1 exist
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        r.vs[0][i] = i < nv ? r.vs[0][i] : 0.f;
        r.vs[1][i] = i + 4 < nv ? r.vs[1][i] : 0.f;
    }
}

template <int D, bool MASKED, bool ALWAYS = false>
__device__ inline void step_update4(TileState<D / 16> &st, const StepRegs4<D> &r, const u32x4_t (&qop)[D / 32],
                                    int kc, const RowVis &rv, int g, float scale_log2, bool fresh = false) {
    float ksc[8], vsc[8];
    step_scales(r, ksc, vsc);
    step_core<D, true, MASKED, ALWAYS>(
        st, [&](int tau, int j) { return fp4x8_to_bf16(r.k[tau][j]); }, [&](int dt) { return fp4x8_to_bf16(r.v[dt]); },
        ksc, vsc, qop, kc, rv, g, scale_log2, fresh);
}

template <int D, bool MASKED>
__device__ inline void step_update4x2(TileState<D / 16> (&st)[2], const StepRegs4<D> &r,
                                      const u32x4_t (&qop)[2][D / 32], int kc, const RowVis (&rv)[2], int g,
                                      float scale_log2) {
    float ksc[8], vsc[8];
    step_scales(r, ksc, vsc);
    step_core2<D, true, MASKED>(
        st, [&](int tau, int j) { return fp4x8_to_bf16(r.k[tau][j]); }, [&](int dt) { return fp4x8_to_bf16(r.v[dt]); },
        ksc, vsc, qop, kc, rv, g, scale_log2);
}

template <int D>
struct Pool<D, kKvFp4> {
    using Regs = StepRegs4<D>;
    static constexpr size_t tile_bytes = (size_t)q4_tile_bytes<D>();
    __device__ static void load(Regs &r, const uint8_t *k0, const uint8_t *v0, const uint8_t *k1, const uint8_t *v1,
                                int g, int n) {
        load_step4<D, false>(r, k0, v0, k1, v1, g, n);
    }
    __device__ static void mask(Regs &r, int kc, int ctx, int g) { mask_tail4<D>(r, kc, ctx, g); }
    template <bool MASKED, bool ALWAYS = false>
    __device__ static void update(TileState<D / 16> &st, const Regs &r, const u32x4_t (&qop)[D / 32], int kc,
                                  const RowVis &rv, int g, float sl2, bool fresh = false) {
        step_update4<D, MASKED, ALWAYS>(st, r, qop, kc, rv, g, sl2, fresh);
    }
    template <bool MASKED>
    __device__ static void update2(TileState<D / 16> (&st)[2], const Regs &r, const u32x4_t (&qop)[2][D / 32], int kc,
                                   const RowVis (&rv)[2], int g, float sl2) {
        step_update4x2<D, MASKED>(st, r, qop, kc, rv, g, sl2);
    }
};

// Rows rho = row0 + 16 t + n of a sequence's [q_len * G] row space, ordered
// r * G + head-in-group.
struct RowInfo {
    int prow;   // last visible key, -1 for padding rows
    int r, hl;  // query row within the sequence, head within the group
};

__device__ inline RowInfo row_info(int rho, int rows_total, int G, int ctx, int q_len) {
    RowInfo ri;
    const bool valid = rho < rows_total;
    ri.r = valid ? rho / G : 0;
    ri.hl = valid ? rho - ri.r * G : 0;
    ri.prow = valid ? ctx - q_len + ri.r : -1;
    return ri;
}

// Visibility of a row (see RowVis); q0 is the sequence's first row, wbase
// the position of its first query row.
template <bool MASKED>
__device__ inline RowVis row_vis(const AttnParams &P, const RowInfo &ri, int q0, int wbase) {
    RowVis v;
    v.prow = ri.prow;
    v.lo = kFarBelow;
    v.wbase = kFarAbove;
    v.tm = 0xFFFFFFFFu;
    if constexpr (MASKED) {
        if (P.window > 0) v.lo = ri.prow - P.window + 1;
        if (P.tree_mask && ri.prow >= 0) {
            v.wbase = wbase;
            v.tm = P.tree_mask[q0 + ri.r] | (1u << ri.r);
        }
    }
    return v;
}

// Lowest position any row of a sequence can see, from its first query row.
__device__ inline int seq_lowest_key(const AttnParams &P, int wbase) {
    return P.window > 0 ? wbase - P.window + 1 : 0;
}

// Q of the lane's row; padding rows read the sequence's first row, which
// they never use (no key is visible to them).
template <int D>
__device__ inline void load_q(u32x4_t (&qop)[D / 32], const AttnParams &P, int q0, const RowInfo &ri, int kvh, int g) {
    const uint16_t *qrow =
        reinterpret_cast<const uint16_t *>(P.q) + ((size_t)(q0 + ri.r) * P.Hq + kvh * P.G + ri.hl) * D;
#pragma unroll
    for (int j = 0; j < D / 32; ++j)
        qop[j] = *reinterpret_cast<const u32x4_t *>(qrow + 32 * j + 8 * g);
}

__device__ inline float sink_log2(const AttnParams &P, int kvh, int hl) {
    return P.sinks ? P.sinks[kvh * P.G + hl] * kLog2e : -INFINITY;
}

template <int DT>
__device__ inline void store_out(const AttnParams &P, int q0, const RowInfo &ri, int kvh, int g, const f32x4_t *o) {
    if (ri.prow < 0) return;
    float *dst = P.out + ((size_t)(q0 + ri.r) * P.Hq + kvh * P.G + ri.hl) * (16 * DT) + 4 * g;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) *reinterpret_cast<f32x4_t *>(dst + 16 * dt) = o[dt];
}

// ---------------------------------------------------------------------------
// Parallel shape: one workgroup per (KV head, sequence, split), in a flat
// grid whose fastest index is the KV head and whose split slots run the
// 1024-key splits before the 256-key ones, so that short workgroups fill the
// end (decode batches whose grid queues: the balanced order below). 4 waves; wave w streams quarter w of the split in 32-key steps for all
// NT tiles (up to 16 NT rows per sequence and KV head). The quarter states
// meet in LDS and wave 0 folds them in order. A sequence whose rows see one
// split only is finished here; otherwise the split state goes to the
// workspace and attn_fold folds the splits.
// (A persistent grid claiming these items from counters, tried as a cure for
// CUs the dispatcher leaves idle, ran slower on every workload measured.)
// ---------------------------------------------------------------------------
__device__ inline int split_of_slot(int z, int max_splits) {
    if (max_splits <= kSplitsA) return z;
    return z + kSplitsA < max_splits ? z + kSplitsA : z - (max_splits - kSplitsA);
}

// Balanced order (decode batches whose grid queues: at most 64 sequences,
// max_splits below 1024, no restricted visibility). The dispatcher deals a
// die's workgroups to its shader engines in turn, by count; a slot order
// fixed in advance hands some engines more keys than others, and slots of
// splits a sequence does not have still take their turn among the busy
// ones. Here every workgroup reads the batch's context lengths (lane l:
// sequence l) and ranks the items by class: the full 1024-key splits (in
// sequence order; a split-major order measured 7-10 % slower), then each
// sequence's partial last split, then the full 256-key splits, then the
// slots past each sequence's splits (which only record an empty state for
// the fold), so that neighbours in dispatch order carry about the same
// number of keys and the short items come last. The price is a round trip:
// the block ids wait for the context lengths. Returns false for a slot past
// all of them. The item computed is the same whichever workgroup takes it.
// Inclusive prefix sum over the 64 lanes of a wave, with DPP: row shifts
// within each row of 16 lanes, then the row totals through the row
// broadcasts of lanes 15 and 31 (no LDS round trip, unlike lane shuffles).
__device__ inline int wave_incl_scan(int x) {
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, true);   // row_shr:1
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, true);   // row_shr:2
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, true);   // row_shr:4
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, true);   // row_shr:8
    x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);  // row_bcast:15 into rows 1, 3
    x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);  // row_bcast:31 into rows 2, 3
    return x;
}

__device__ inline bool balanced_item(const AttnParams &P, int rank, int cap_rows, int lane, int &s, int &j, int &ctx,
                                     int &qa, int &qb) {
    const bool in = lane < P.num_seqs;
    const int c = in ? P.ctx_lens[lane] : 0;
    const int a = P.decode_only ? lane : (in ? P.qsl[lane] : 0);
    const int b = P.decode_only ? lane + 1 : (in ? P.qsl[lane + 1] : 0);
    const int ql = b - a, rows = ql * P.G;
    const int pmax = c - ql + (rows - 1) / P.G;
    // the sequences the parallel shape takes (the same test as its items')
    const bool ok = in && a >= 0 && ql > 0 && b <= P.total_rows && rows <= cap_rows && pmax >= 0;
    const int ns = ok ? min(num_splits(pmax + 1), P.max_splits) : 0;
    const int part = ns > 0 && split_begin(ns) > pmax + 1;  // its last split is partial
    const int nA = max(ns - kSplitsA, 0) - (part && ns > kSplitsA ? 1 : 0);
    const int nB = min(ns, kSplitsA) - (part && ns <= kSplitsA ? 1 : 0);
    const int nE = ok ? P.max_splits - ns : 0;
    // inclusive scans over the lanes, two 16-bit counts per word
    const int v0 = nA | (nE << 16), v1 = part | (nB << 16);
    const int i0 = wave_incl_scan(v0), i1 = wave_incl_scan(v1);
    const int t0 = __builtin_amdgcn_readlane(i0, 63), t1 = __builtin_amdgcn_readlane(i1, 63);
    const int NA = t0 & 0xffff, NE = t0 >> 16, NP = t1 & 0xffff, NB = t1 >> 16;
    int r = rank, cls, hi, cnt;
    if (r < NA) {
        cls = 0, hi = i0 & 0xffff, cnt = nA;
    } else if ((r -= NA) < NP) {
        cls = 1, hi = i1 & 0xffff, cnt = part;
    } else if ((r -= NP) < NB) {
        cls = 2, hi = i1 >> 16, cnt = nB;
    } else if ((r -= NB) < NE) {
        cls = 3, hi = i0 >> 16, cnt = nE;
    } else {
        return false;
    }
    const unsigned long long hit = __ballot(cnt > 0 && hi - cnt <= r && r < hi);  // one lane
    if (!hit) return false;
    const int l = __ffsll((long long)hit) - 1;
    const int off = r - __builtin_amdgcn_readlane(hi - cnt, l);
    const int ns_l = __builtin_amdgcn_readlane(ns, l);
    s = l;
    j = cls == 0 ? kSplitsA + off : cls == 1 ? ns_l - 1 : cls == 2 ? off : ns_l + off;
    ctx = __builtin_amdgcn_readlane(c, l);
    qa = __builtin_amdgcn_readlane(a, l);
    qb = __builtin_amdgcn_readlane(b, l);
    return true;
}

// Waves per SIMD the parallel shape is built for: the register budget that
// keeps enough workgroups resident to cover load latency. The two-stage
// variant (PF) serves grids that leave CUs free, where occupancy does not
// matter, and takes the whole register file.
constexpr int par_waves(int D, int NT, bool PF) {
    return PF ? 2 : D == 64 ? (NT == 1 ? 5 : 3) : (NT == 1 ? 3 : 2);
}

template <int D, int NT>
struct ParLds {
    f32x4_t acc[3][NT][D / 16][64];
    float2 ml[3][NT][64];
};


// Slot order of a grid with a shared prefix, per KV head (rest = blockIdx /
// Hkv), longest items first:
//   group items of the prefix's 1024-key splits  (g fastest),
//   the prefix sequences' own splits from pre_splits on (s fastest),
//   every split of the other sequences             (s fastest, split_of_slot),
//   group items of the prefix's 256-key splits    (g fastest).
// Returns 1 for a group item (s = its group), 0 for a sequence's split, -1
// past the grid.
__device__ inline int prefix_slot(const AttnParams &P, int rest, int &s, int &j) {
    const int js = min(P.pre_splits, kSplitsA), jl = P.pre_splits - js;
    int r = rest;
    if (r < P.pre_groups * jl) {
        s = r % P.pre_groups;
        j = kSplitsA + r / P.pre_groups;
        return 1;
    }
    r -= P.pre_groups * jl;
    if (r < P.pre_a) {
        s = r % P.pre_seqs;
        j = P.pre_splits + r / P.pre_seqs;
        return 0;
    }
    r -= P.pre_a;
    const int others = P.num_seqs - P.pre_seqs;
    if (r < others * P.max_splits) {
        s = P.pre_seqs + r % others;
        j = split_of_slot(r / others, P.max_splits);
        return 0;
    }
    r -= others * P.max_splits;
    if (r < P.pre_groups * js) {
        s = r % P.pre_groups;
        j = r / P.pre_groups;
        return 1;
    }
    return -1;
}

// One group item: split j of the prefix sequences g * pre_m .. + pre_m - 1,
// all of them decode rows whose keys of the split lie in the same physical
// blocks. Wave w streams quarter w once, for a tile holding every member's
// rows (member m's head hl at tile row m * G + hl): the bits of each row are
// those of the row alone, since an MFMA's per-element results do not depend
// on the other rows of its tile and every row is masked by its own position.
// The block ids are checked: if any quarter of the split is not the same
// physical blocks for every member, or a member has more than one row, the
// workgroup computes the members one after another over their own blocks
// (the rows of a member with more than 32 rows are the prefill shape's).
template <int D, int KF>
__device__ void prefix_group_item(const AttnParams &P, int kvh, int grp, int j, int wave, int lane,
                                  ParLds<D, 1> &lds) {
    using PoolT = Pool<D, KF>;
    using Regs = typename PoolT::Regs;
    constexpr int DT = D / 16, KJ = D / 32;
    const int g = lane >> 4, n = lane & 15;
    const int s0 = grp * P.pre_m;
    const int nm = min(P.pre_m, P.pre_seqs - s0);
    // member metadata (lane m) and block ids (lane 16 m + i: block i of the
    // wave's quarter of member m), one round trip
    const int ks = split_begin(j);
    const int ql = (split_begin(j + 1) - ks) >> 2;
    const int kq0 = ks + wave * ql;
    const int nqb = ql / kBlock;  // blocks per quarter (4 or 16)
    int mc = 0, ma = 0, mb = 0;
    if (lane < nm) {
        mc = P.ctx_lens[s0 + lane];
        ma = P.qsl[s0 + lane];
        mb = P.qsl[s0 + lane + 1];
    }
    int bidm = -1, bid3 = -1;  // bid3: the same for the split's last quarter
    {
        const int m = lane >> 4, i = lane & 15;
        if (m < nm && i < nqb) {
            const int jb = kq0 / kBlock + i;
            const int b = P.bt[(size_t)(s0 + m) * P.max_blocks_per_seq + min(jb, P.max_blocks_per_seq - 1)];
            bidm = (jb < P.max_blocks_per_seq && b >= 0 && b < P.num_blocks) ? b : -1;
            const int jb3 = (ks + 3 * ql) / kBlock + i;
            const int b3 = P.bt[(size_t)(s0 + m) * P.max_blocks_per_seq + min(jb3, P.max_blocks_per_seq - 1)];
            bid3 = (jb3 < P.max_blocks_per_seq && b3 >= 0 && b3 < P.num_blocks) ? b3 : -1;
        }
    }
    // shared: every member one decode row whose context holds the whole
    // quarter, and the same valid block ids as member 0
    bool ok = true, singles = true;
    for (int m = 0; m < nm; ++m) {
        const int c = __builtin_amdgcn_readlane(mc, m);
        const int a = __builtin_amdgcn_readlane(ma, m), b = __builtin_amdgcn_readlane(mb, m);
        singles = singles && b - a == 1 && a >= 0 && b <= P.total_rows;
        ok = ok && c >= kq0 + ql;
    }
    ok = ok && singles;
    const int lead = __shfl(bidm, lane & 15, 64);
    const bool mine = (lane >> 4) < nm && (lane & 15) < nqb;
    ok = ok && !__any(mine && (bidm < 0 || bidm != lead));
    __shared__ int s_ok[4];
    if (lane == 0) s_ok[wave] = ok;
    __syncthreads();
    const bool shared = s_ok[0] && s_ok[1] && s_ok[2] && s_ok[3];
    // the split that holds the prefix's end: its first three quarters shared,
    // the last not (every member one decode row)
    const bool last_only = !shared && s_ok[0] && s_ok[1] && s_ok[2] && singles;

    const size_t tile = PoolT::tile_bytes;
    const uint8_t *kbase = reinterpret_cast<const uint8_t *>(P.kp) + (size_t)kvh * tile;
    const uint8_t *vbase = reinterpret_cast<const uint8_t *>(P.vp) + (size_t)kvh * tile;
    const uint8_t *zero = reinterpret_cast<const uint8_t *>(g_zero_tile);
    const size_t bstride = (size_t)P.Hkv * tile;

    // One pass: the rows of the tile (per lane: q row, head, position, or
    // prow -1 for no row), the member whose block ids the keys come from
    // (lanes 16 src ..) and its context length; writes each row's split state.
    auto pass = [&](int qrow, int hl, int prow, int src, int ctx) {
        RowInfo ri;
        ri.r = 0;
        ri.hl = hl;
        ri.prow = prow;
        RowVis rv;
        rv.prow = prow;
        rv.lo = kFarBelow;
        rv.wbase = kFarAbove;
        rv.tm = 0xFFFFFFFFu;
        u32x4_t qop[KJ];
        load_q<D>(qop, P, qrow, ri, kvh, g);  // row qrow + r, r = 0
        TileState<DT> st;
        state_clear(st);
        const int kq1 = min(kq0 + ql, ctx);
        for (int kc = kq0; kc < kq1; kc += kStep) {
            const int li = src * 16 + (kc - kq0) / kBlock;
            const int b0 = __builtin_amdgcn_readlane(bidm, li);
            const int b1 = __builtin_amdgcn_readlane(bidm, li + 1);
            Regs r;
            PoolT::load(r, b0 >= 0 ? kbase + (size_t)b0 * bstride : zero, b0 >= 0 ? vbase + (size_t)b0 * bstride : zero,
                        b1 >= 0 ? kbase + (size_t)b1 * bstride : zero, b1 >= 0 ? vbase + (size_t)b1 * bstride : zero,
                        g, n);
            PoolT::mask(r, kc, ctx, g);
            PoolT::template update<false>(st, r, qop, kc, rv, g, P.scale_log2);
        }
        if (wave > 0) {
            lds.ml[wave - 1][0][lane] = make_float2(st.m, st.l);
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) lds.acc[wave - 1][0][dt][lane] = st.acc[dt];
        }
        __syncthreads();
        if (wave == 0 && prow >= 0) {
#pragma unroll
            for (int w = 0; w < 3; ++w) {
                TileState<DT> o;
                const float2 ml = lds.ml[w][0][lane];
                o.m = ml.x;
                o.l = ml.y;
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) o.acc[dt] = lds.acc[w][0][dt][lane];
                fold_state(st, o);
            }
            const size_t base = ((size_t)qrow * P.Hq + kvh * P.G + hl) * P.max_splits + j;
            if (g == 0) P.ws_ml[base] = make_float2(st.m, st.l);
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
                *reinterpret_cast<f32x4_t *>(P.ws_acc + base * D + 16 * dt + 4 * g) = st.acc[dt];
        }
        __syncthreads();  // wave 0 has read the LDS states before the next pass writes them
    };

    // One quarter [qa, qa + ql) of a tile (rows as in pass), keys from member
    // src's block ids held in bids (lane 16 src + i), into st.
    auto quarter = [&](int qrow, int hl, int prow, int src, int ctx, int qa, int bids, TileState<DT> &st) {
        RowInfo ri;
        ri.r = 0;
        ri.hl = hl;
        ri.prow = prow;
        RowVis rv;
        rv.prow = prow;
        rv.lo = kFarBelow;
        rv.wbase = kFarAbove;
        rv.tm = 0xFFFFFFFFu;
        u32x4_t qop[KJ];
        load_q<D>(qop, P, qrow, ri, kvh, g);
        state_clear(st);
        const int kq1 = min(qa + ql, ctx);
        for (int kc = qa; kc < kq1; kc += kStep) {
            const int li = src * 16 + (kc - qa) / kBlock;
            const int b0 = __builtin_amdgcn_readlane(bids, li);
            const int b1 = __builtin_amdgcn_readlane(bids, li + 1);
            Regs r;
            PoolT::load(r, b0 >= 0 ? kbase + (size_t)b0 * bstride : zero, b0 >= 0 ? vbase + (size_t)b0 * bstride : zero,
                        b1 >= 0 ? kbase + (size_t)b1 * bstride : zero, b1 >= 0 ? vbase + (size_t)b1 * bstride : zero,
                        g, n);
            PoolT::mask(r, kc, ctx, g);
            PoolT::template update<false>(st, r, qop, kc, rv, g, P.scale_log2);
        }
    };

    if (last_only) {
        // Waves 0-2 stream their quarter once for the group tile (member m's
        // head hl at tile row m * G + hl); the members' last quarters, over
        // their own blocks with only that member's rows seeing keys, go to
        // waves 3, 3, 1, 2 (members 0-3), so that no wave streams more than
        // two quarters. Member rows keep the tile's layout, and every row's
        // quarter states meet in quarter order, as in the row alone.
        const int m_row = n / P.G, hl = n - m_row * P.G;
        const bool row = m_row < nm && n < nm * P.G;
        const int mm = row ? m_row : 0;
        int a = 0, c = 0;
        for (int k = 0; k < nm; ++k)
            if (mm == k) {
                a = __builtin_amdgcn_readlane(ma, k);
                c = __builtin_amdgcn_readlane(mc, k);
            }
        int cmax = 0;
        for (int k = 0; k < nm; ++k) cmax = max(cmax, __builtin_amdgcn_readlane(mc, k));
        TileState<DT> st;
        state_clear(st);
        if (wave < 3) {
            quarter(a, row ? hl : 0, row ? c - 1 : -1, 0, cmax, kq0, bidm, st);
            if (wave > 0) {
                lds.ml[wave - 1][0][lane] = make_float2(st.m, st.l);
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) lds.acc[wave - 1][0][dt][lane] = st.acc[dt];
            }
        }
        // (wave 0 takes no member: its quarter state stays in st for the fold,
        // and the other waves reuse st, whose state is in LDS by now)
        for (int m = 0; m < nm; ++m) {
            if ((m < 2 ? 3 : m - 1) != wave) continue;  // uniform over the wave
            const int cm = __builtin_amdgcn_readlane(mc, m), am = __builtin_amdgcn_readlane(ma, m);
            const bool mine_row = row && m_row == m;
            quarter(am, mine_row ? hl : 0, mine_row ? cm - 1 : -1, m, cm, ks + 3 * ql, bid3, st);
            if (mine_row) {
                lds.ml[2][0][lane] = make_float2(st.m, st.l);
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) lds.acc[2][0][dt][lane] = st.acc[dt];
            }
        }
        __syncthreads();
        if (wave == 0 && row) {
#pragma unroll
            for (int w = 0; w < 3; ++w) {
                TileState<DT> o;
                const float2 ml = lds.ml[w][0][lane];
                o.m = ml.x;
                o.l = ml.y;
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) o.acc[dt] = lds.acc[w][0][dt][lane];
                fold_state(st, o);
            }
            const size_t base = ((size_t)a * P.Hq + kvh * P.G + hl) * P.max_splits + j;
            if (g == 0) P.ws_ml[base] = make_float2(st.m, st.l);
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
                *reinterpret_cast<f32x4_t *>(P.ws_acc + base * D + 16 * dt + 4 * g) = st.acc[dt];
        }
        return;
    }

    if (shared) {
        const int m = n / P.G, hl = n - m * P.G;
        const bool row = m < nm && n < nm * P.G;
        const int mm = row ? m : 0;
        // one readlane per member (nm <= 4), so that no lane indexes a register
        int a = 0, c = 0;
        for (int k = 0; k < nm; ++k)
            if (mm == k) {
                a = __builtin_amdgcn_readlane(ma, k);
                c = __builtin_amdgcn_readlane(mc, k);
            }
        int cmax = 0;
        for (int k = 0; k < nm; ++k) cmax = max(cmax, __builtin_amdgcn_readlane(mc, k));
        pass(a, row ? hl : 0, row ? c - 1 : -1, 0, cmax);
    } else {
        for (int m = 0; m < nm; ++m) {
            const int c = __builtin_amdgcn_readlane(mc, m);
            const int a = __builtin_amdgcn_readlane(ma, m), b = __builtin_amdgcn_readlane(mb, m);
            const int q_len = b - a, rows = q_len * P.G;
            if (!(a >= 0 && q_len > 0 && b <= P.total_rows && rows <= kParRows && c - q_len >= 0)) continue;
            for (int p0 = 0; p0 < rows; p0 += 16) {
                const int rho = p0 + n;
                const bool row = rho < rows;
                const int r = row ? rho / P.G : 0, hl = row ? rho - (rho / P.G) * P.G : 0;
                pass(a + r, hl, row ? c - q_len + r : -1, m, c);
            }
        }
    }
}

// TWO: one-tile instances that also take sequences of 17 to 32 rows, in two
// passes of 16 rows over the same keys (quantized batches with prefill
// chunks, so that one launch covers decode and verify rows).
// PREFIX: the instances of paged_attention_prefix_forward (one tile,
// unmasked, no append), whose grid is prefix_slot's.
template <int D, int NT, bool PF, bool APPEND, int KF, bool MASKED, bool TWO = false, bool PREFIX = false>
__global__ __launch_bounds__(256, par_waves(D, NT, PF) - ((TWO || PREFIX) && D == 64 ? 1 : 0)) void attn_parallel(
    AttnParams P) {
    constexpr int NPASS = TWO ? 2 : 1;
    using PoolT = Pool<D, KF>;
    using Regs = typename PoolT::Regs;
    constexpr int DT = D / 16, KJ = D / 32;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;  // wave index is uniform
    const int g = lane >> 4, n = lane & 15;
    const int kvh = blockIdx.x % P.Hkv;
    const int rest = blockIdx.x / P.Hkv;
    __shared__ ParLds<D, NT> lds;  // quarter states of waves 1-3
    int s, j, ctx, qa, qb;
    static_assert(!PREFIX || (NT == 1 && !APPEND && !MASKED), "prefix instances: one tile, unmasked, no append");
    if constexpr (PREFIX) {
        const int kind = prefix_slot(P, rest, s, j);
        if (kind < 0) return;
        if (kind == 1) {
            prefix_group_item<D, KF>(P, kvh, s, j, wave, lane, lds);
            return;
        }
        ctx = P.ctx_lens[s];
        qa = P.qsl[s];
        qb = P.qsl[s + 1];
    } else if (!MASKED && P.seq_stride == 0) {
        if (!balanced_item(P, rest, 16 * NT * NPASS, lane, s, j, ctx, qa, qb)) return;
    } else {
        s = rest % P.seq_stride;
        j = split_of_slot(rest / P.seq_stride, P.max_splits);
        if (s >= P.num_seqs) return;  // padding slot
        // Loads that need nothing but the grid position go out together: the
        // context length, the row offsets, and the block ids of the wave's
        // quarter (below). (no branches among them, so that none waits for another)
        ctx = P.ctx_lens[s];
        qa = P.qsl[s];
        qb = P.qsl[s + 1];
    }
    if constexpr (MASKED) {
        if (P.grid_splits < P.max_splits) {  // grid slot z: the z-th split from the lowest visible key's
            j = split_index(max(ctx - (P.decode_only ? 1 : qb - qa) - P.window + 1, 0)) + rest / P.seq_stride;
            if (j >= P.max_splits) return;
        }
    }
    // the block ids of the wave's quarter [kq0, kq0 + ql), lane i holding
    // block kq0/16 + i
    const int ks = split_begin(j);
    const int ql = (split_begin(j + 1) - ks) >> 2;
    const int kq0 = ks + wave * ql;
    const int jb = kq0 / kBlock + lane;
    int bid = P.bt[(size_t)s * P.max_blocks_per_seq + min(jb, P.max_blocks_per_seq - 1)];
    const int q0 = P.decode_only ? s : qa;
    const int q_len = P.decode_only ? 1 : qb - qa;

    const int rows_total = q_len * P.G;
    const int p_max = ctx - q_len + (rows_total - 1) / P.G;
    const int ns_item = min(num_splits(p_max + 1), P.max_splits);
    // (uniform over the workgroup)
    if (!(q0 >= 0 && q_len > 0 && q0 + q_len <= P.total_rows && rows_total <= 16 * NT * NPASS && p_max >= 0))
        return;
    const int wbase = ctx - q_len;                              // position of the first query row
    const int lo_seq = MASKED ? seq_lowest_key(P, wbase) : 0;  // no row sees a key below it
    if (j >= ns_item || (MASKED && split_begin(j + 1) <= lo_seq)) {
        // No row sees this split: its slot holds an empty state, so that the
        // fold reads every slot without first learning the context length.
        if (wave == 0) {
#pragma unroll
            for (int t = 0; t < NT * NPASS; ++t) {
                const int rho = 16 * t + n;
                if (g != 0 || rho >= rows_total) continue;
                const int r = rho / P.G, hl = rho - r * P.G;
                P.ws_ml[((size_t)(q0 + r) * P.Hq + kvh * P.G + hl) * P.max_splits + j] = make_float2(-INFINITY, 0.f);
            }
        }
        return;
    }
    for (int pass = 0; pass < NPASS; ++pass) {
        if (TWO && 16 * NT * pass >= rows_total) break;  // uniform
        RowInfo ri[NT];
        RowVis rv[NT];
        u32x4_t qop[NT][KJ];
        TileState<DT> st[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            state_clear(st[t]);
            ri[t] = row_info(16 * (NT * pass + t) + n, rows_total, P.G, ctx, q_len);
            rv[t] = row_vis<MASKED>(P, ri[t], q0, wbase);
        }
        {
#pragma unroll
            for (int t = 0; t < NT; ++t) load_q<D>(qop[t], P, q0, ri[t], kvh, g);
            const int kq1 = min(kq0 + ql, p_max + 1);
            bid = (lane < ql / kBlock && jb < (ctx + kBlock - 1) / kBlock && jb < P.max_blocks_per_seq && bid >= 0 &&
                   bid < P.num_blocks)
                      ? bid
                      : -1;
            // appending decode step: the wave whose quarter holds the new key
            const int pn = ctx - 1;
            const bool fused = APPEND && KF == kKvBf16 && kq0 <= pn && pn < kq1;
            // The new token's K and V rows wait in LDS (this wave's slot) for the
            // step that holds pn, rather than in registers through the loop.
            // Staged after the wave's first K/V loads are issued, so that the
            // two round trips overlap.
            __shared__ __attribute__((aligned(16))) uint16_t s_new[APPEND ? 4 : 1][2][D];
            auto stage_new = [&]() {
            if (APPEND && KF == kKvBf16 && fused) {
                const size_t rowoff = ((size_t)s * P.Hkv + kvh) * D;
                const int slot = P.slots[s];
                if (lane < D / 8) {
                    const u32x4_t kq = *reinterpret_cast<const u32x4_t *>(P.k_new + rowoff + lane * 8);
                    *reinterpret_cast<u32x4_t *>(&s_new[wave][0][lane * 8]) = kq;
                    *reinterpret_cast<u32x4_t *>(&s_new[wave][1][lane * 8]) =
                        *reinterpret_cast<const u32x4_t *>(P.v_new + rowoff + lane * 8);
                    // and writes it to its pool slot, as the scatter-write would
                    if (slot >= 0 && slot < P.num_blocks * kBlock) {
                        const size_t tb = ((size_t)(slot / kBlock) * P.Hkv + kvh) * D;  // element offset of the tile
                        *reinterpret_cast<u32x4_t *>(P.kp_w + tb * kBlock + ((size_t)lane * kBlock + slot % kBlock) * 8) =
                            kq;
                    }
                }
                if (slot >= 0 && slot < P.num_blocks * kBlock) {
                    const size_t tb = ((size_t)(slot / kBlock) * P.Hkv + kvh) * D;
#pragma unroll
                    for (int c = lane; c < D; c += 64)
                        P.vp_w[tb * kBlock + (size_t)c * kBlock + slot % kBlock] = P.v_new[rowoff + c];
                }
            }
            };
            const size_t tile = PoolT::tile_bytes;
            const uint8_t *kbase = reinterpret_cast<const uint8_t *>(P.kp) + (size_t)kvh * tile;
            const uint8_t *vbase = reinterpret_cast<const uint8_t *>(P.vp) + (size_t)kvh * tile;
            const uint8_t *zero = reinterpret_cast<const uint8_t *>(g_zero_tile);
            const size_t bstride = (size_t)P.Hkv * tile;
            // Step at key kc; lanes past the quarter's blocks hold -1, so a fetch
            // one step past the end reads the zero tile.
            auto fetch = [&](Regs &r, int kc) {
                const int li = (kc - kq0) / kBlock;
                const int b0 = __builtin_amdgcn_readlane(bid, li);
                const int b1 = __builtin_amdgcn_readlane(bid, li + 1);
                PoolT::load(r, b0 >= 0 ? kbase + (size_t)b0 * bstride : zero, b0 >= 0 ? vbase + (size_t)b0 * bstride : zero,
                            b1 >= 0 ? kbase + (size_t)b1 * bstride : zero, b1 >= 0 ? vbase + (size_t)b1 * bstride : zero,
                            g, n);
            };
            auto compute = [&](Regs &r, int kc) {
                if constexpr (APPEND && KF == kKvBf16) {
                    if (fused && kc <= pn && pn < kc + kStep) {
                        // LDS operations of one wave complete in order: the rows
                        // written above are there
                        u32x4_t knew[KJ];
                        uint32_t vnew[DT];
#pragma unroll
                        for (int jj = 0; jj < KJ; ++jj)
                            knew[jj] = *reinterpret_cast<const u32x4_t *>(&s_new[wave][0][(4 * jj + g) * 8]);
#pragma unroll
                        for (int dt = 0; dt < DT; ++dt) vnew[dt] = s_new[wave][1][16 * dt + n];
                        patch_new_key<D>(r, knew, vnew, kc, pn, g, n);
                    }
                }
                PoolT::mask(r, kc, ctx, g);
                if constexpr (NT == 2) {
                    if (rows_total > 16)  // uniform: both tiles in one pass over the operands
                        PoolT::template update2<MASKED>(st, r, qop, kc, rv, g, P.scale_log2);
                    else
                        PoolT::template update<MASKED>(st[0], r, qop[0], kc, rv[0], g, P.scale_log2);
                } else {
#pragma unroll
                    for (int t = 0; t < NT; ++t)
                        if (16 * t < rows_total)
                            PoolT::template update<MASKED>(st[t], r, qop[t], kc, rv[t], g, P.scale_log2);
                }
            };
            // Steps wholly below every row's lowest visible key change no state:
            // the wave starts at the step holding lo_seq.
            const int kstart = (MASKED && lo_seq > kq0) ? kq0 + (lo_seq - kq0) / kStep * kStep : kq0;
            if constexpr (PF) {
                // Two register stages, each refilled as soon as it is consumed,
                // so that two steps are in flight; unrolled so that each stage
                // keeps fixed registers (a copy between stages would wait for the
                // loads it copies).
                Regs r0, r1;
                if (!MASKED || kstart < kq1) fetch(r0, kstart);
                if (kstart + kStep < kq1) fetch(r1, kstart + kStep);
                stage_new();
                for (int kc = kstart; kc < kq1; kc += 2 * kStep) {
                    compute(r0, kc);
                    if (kc + 2 * kStep < kq1) fetch(r0, kc + 2 * kStep);
                    if (kc + kStep < kq1) {
                        compute(r1, kc + kStep);
                        if (kc + 3 * kStep < kq1) fetch(r1, kc + 3 * kStep);
                    }
                }
            } else {
                for (int kc = kstart; kc < kq1; kc += kStep) {
                    Regs r;
                    fetch(r, kc);
                    if (kc == kstart) stage_new();  // (a fused quarter holds pn, so it has a step)
                    compute(r, kc);
                }
            }
        }
        if (wave > 0) {
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                lds.ml[wave - 1][t][lane] = make_float2(st[t].m, st[t].l);
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) lds.acc[wave - 1][t][dt][lane] = st[t].acc[dt];
            }
        }
        __syncthreads();
        if (wave != 0) {
            if constexpr (!TWO) return;
            __syncthreads();  // wave 0 has read the LDS states before the next pass writes them
            continue;
        }
        // quarter states -> split state (left fold in quarter order); with one
        // split slot there is no fold launch and the rows are finished here
        const bool whole = P.max_splits == 1;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            if (ri[t].prow < 0) continue;
#pragma unroll
            for (int w = 0; w < 3; ++w) {
                TileState<DT> o;
                const float2 ml = lds.ml[w][t][lane];
                o.m = ml.x;
                o.l = ml.y;
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) o.acc[dt] = lds.acc[w][t][dt][lane];
                fold_state(st[t], o);
            }
            if (whole) {
                f32x4_t o[DT];
                finalize(st[t], sink_log2(P, kvh, ri[t].hl), o);
                store_out<DT>(P, q0, ri[t], kvh, g, o);
            } else {
                const size_t base = ((size_t)(q0 + ri[t].r) * P.Hq + kvh * P.G + ri[t].hl) * P.max_splits + j;
                if (g == 0) P.ws_ml[base] = make_float2(st[t].m, st[t].l);
#pragma unroll
                for (int dt = 0; dt < DT; ++dt)
                    *reinterpret_cast<f32x4_t *>(P.ws_acc + base * D + 16 * dt + 4 * g) = st[t].acc[dt];
            }
        }
        if constexpr (TWO) __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// Split fold of the parallel shape: grid (sequence, KV head, group of cells),
// a cell being one (query row, query head) of the sequence's rows for that KV
// head. D / 4 lanes hold a cell's accumulator, four consecutive channels each,
// so every load and store covers whole cache lines; the fold is elementwise in
// d and every lane of a cell repeats the same m, l fold. The split states are
// folded left to right, sixteen per round trip, then finalized.
// ---------------------------------------------------------------------------
// WIDE: the instance for rows of 17 to 32 split slots (launched when the
// batch has that many), whose registers the others do not pay for.
template <int D, int NT, bool WIDE = false>
__global__ __launch_bounds__(256) void attn_fold(AttnParams P) {
    constexpr int LPC = D / 4;         // lanes per cell
    constexpr int CPG = 256 / LPC;     // cells per workgroup
    static_assert(D % 64 == 0, "head_dim must be a multiple of 64");
    const int tid = threadIdx.x;
    const int s = blockIdx.x, kvh = blockIdx.y;
    const int cell = blockIdx.z * CPG + tid / LPC;  // rho = r * G + hl within the sequence
    const int e = (tid % LPC) * 4;                  // the lane's first channel
    // Every kernel argument the fold reads, in scalar registers before the
    // first branch: one round trip for all of them (a workgroup per CU meets
    // a cold scalar cache) instead of one after each branch.
    asm volatile("" ::"s"(P.decode_only), "s"(P.G), "s"(P.total_rows), "s"(P.Hq), "s"(P.max_splits),
                 "s"(P.grid_splits), "s"(P.window), "s"(P.qsl), "s"(P.ctx_lens), "s"(P.ws_ml), "s"(P.ws_acc),
                 "s"(P.out), "s"(P.sinks));
    int q0, q_len;
    if (P.decode_only) {
        q0 = s;
        q_len = 1;
    } else {
        q0 = P.qsl[s];
        q_len = P.qsl[s + 1] - q0;
    }
    const int rows_total = q_len * P.G;
    if (q0 < 0 || q_len <= 0 || q0 + q_len > P.total_rows || rows_total > 16 * NT || cell >= rows_total) return;
    // every slot holds a state (empty past the row's keys): no context length needed
    const int r = cell / P.G, hl = cell - r * P.G;
    const size_t base0 = ((size_t)(q0 + r) * P.Hq + kvh * P.G + hl) * P.max_splits;
    float m = -INFINITY, l = 0.f;
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    // the slots the parallel grid wrote (all, or a sliding window's run)
    int j0 = 0, j1 = P.max_splits;
    if (P.grid_splits < P.max_splits) {
        j0 = split_index(max(P.ctx_lens[s] - q_len - P.window + 1, 0));
        j1 = min(j0 + P.grid_splits, P.max_splits);
    }
    constexpr int U = 16;
    if (WIDE && j1 - j0 > U && j1 - j0 <= 2 * U) {
        // Two round trips either way: the (m, l) of every slot first, then
        // the accumulators of the slots that hold a state (an empty slot's
        // were never written).
        float2 xml[2 * U];
        f32x4_t xacc[2 * U];
#pragma unroll
        for (int u = 0; u < 2 * U; ++u) xml[u] = j0 + u < j1 ? P.ws_ml[base0 + j0 + u] : make_float2(-INFINITY, 0.f);
#pragma unroll
        for (int u = 0; u < 2 * U; ++u) {
            xacc[u] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            if (xml[u].x != -INFINITY) xacc[u] = *reinterpret_cast<const f32x4_t *>(P.ws_acc + (base0 + j0 + u) * D + e);
        }
#pragma unroll
        for (int u = 0; u < 2 * U; ++u) {
            if (xml[u].x == -INFINITY) continue;
            if (m == -INFINITY) {
                m = xml[u].x;
                l = xml[u].y;
                acc = xacc[u];
                continue;
            }
            const float M = fmaxf(m, xml[u].x);
            const float al = fast_exp2(m - M);
            const float be = fast_exp2(xml[u].x - M);
            l = fmaf(l, al, xml[u].y * be);
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[i] = fmaf(acc[i], al, xacc[u][i] * be);
            m = M;
        }
        j0 = j1;  // done
    }
    // sixteen split states per round trip
    for (int j = j0; j < j1; j += U) {
        float2 xml[U];
        f32x4_t xacc[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            xml[u] = make_float2(-INFINITY, 0.f);
            xacc[u] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            if (j + u < j1) {
                xml[u] = P.ws_ml[base0 + j + u];
                xacc[u] = *reinterpret_cast<const f32x4_t *>(P.ws_acc + (base0 + j + u) * D + e);
            }
        }
        // the fold of two states (as fold_state, element by element)
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (xml[u].x == -INFINITY) continue;
            if (m == -INFINITY) {
                m = xml[u].x;
                l = xml[u].y;
                acc = xacc[u];
                continue;
            }
            const float M = fmaxf(m, xml[u].x);
            const float al = fast_exp2(m - M);
            const float be = fast_exp2(xml[u].x - M);
            l = fmaf(l, al, xml[u].y * be);
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[i] = fmaf(acc[i], al, xacc[u][i] * be);
            m = M;
        }
    }
    TileState<1> st;
    st.m = m;
    st.l = l;
    st.acc[0] = acc;
    f32x4_t o[1];
    finalize(st, sink_log2(P, kvh, hl), o);
    *reinterpret_cast<f32x4_t *>(P.out + ((size_t)(q0 + r) * P.Hq + kvh * P.G + hl) * D + e) = o[0];
}

// ---------------------------------------------------------------------------
// Sequential shape: one workgroup per 64 rows (4 tiles, wave w owns tile w)
// of a sequence with more than kParRows rows per KV head. The workgroup walks
// every chunk up to its last row's position; all 256 threads stage each
// chunk's K/V in LDS, and each wave folds quarters and splits in registers.
// ---------------------------------------------------------------------------
__device__ inline bool find_seq_item(const int32_t *qsl, int S, int G, int item, int lane, int &s_out, int &rb_out) {
    int base = 0;
    for (int t0 = 0; t0 < S; t0 += 64) {
        const int t = t0 + lane;
        int nb = 0;
        if (t < S) {
            const int rows = (qsl[t + 1] - qsl[t]) * G;
            nb = rows > kParRows ? (rows + kSeqRows - 1) / kSeqRows : 0;
        }
        const int incl = wave_incl_scan(nb);
        const int excl = incl - nb;
        const bool hit = t < S && item >= base + excl && item < base + incl;
        const unsigned long long mask = __ballot(hit);
        if (mask) {
            const int l = __ffsll((long long)mask) - 1;
            s_out = t0 + l;
            // row blocks in reverse: under the causal mask the last rows see
            // the most keys, and the longest workgroups should start first
            rb_out = __shfl(nb, l, 64) - 1 - (item - base - __shfl(excl, l, 64));
            return true;
        }
        base += __shfl(incl, 63, 64);
    }
    return false;
}

// Two workgroups per CU (the LDS staging allows no more): bounding the
// registers to that occupancy keeps the MFMA accumulators in VGPRs, where the
// per-step rescale and MFMA accumulation use them without copies.
template <int D, int KF, bool MASKED>
__global__ __launch_bounds__(256, 2) void attn_sequential(AttnParams P) {
    using PoolT = Pool<D, KF>;
    using Regs = typename PoolT::Regs;
    constexpr int DT = D / 16, KJ = D / 32;
    constexpr int TB = (int)PoolT::tile_bytes;  // bytes of one (block, head) tile
    constexpr int NP = TB / 16;                 // its 16-byte pieces
    constexpr int NV = (NP + 63) / 64;          // pieces each lane stages (lane + 64 v)
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;  // wave index is uniform
    const int g = lane >> 4, n = lane & 15;
    const int kvh = blockIdx.x % P.Hkv;  // heads fastest: each row block's heads start together

    int s = 0, rb = 0;
    if (!find_seq_item(P.qsl, P.num_seqs, P.G, blockIdx.x / P.Hkv, lane, s, rb)) return;
    // uniform (a ballot's lane and values broadcast from it): in scalar
    // registers, the walk below and its boundary tests stay scalar too
    s = __builtin_amdgcn_readfirstlane(s);
    rb = __builtin_amdgcn_readfirstlane(rb);
    const int q0 = P.qsl[s];
    const int q_len = P.qsl[s + 1] - q0;
    const int ctx = P.ctx_lens[s];
    const int rows_total = q_len * P.G;
    if (q0 < 0 || q_len <= 0 || q0 + q_len > P.total_rows) return;
    const int row0 = rb * kSeqRows;
    const int row_last = min(row0 + kSeqRows, rows_total) - 1;
    const int p_max = ctx - q_len + row_last / P.G;
    if (p_max < 0) return;

    const RowInfo ri = row_info(row0 + 16 * wave + n, rows_total, P.G, ctx, q_len);
    const RowVis rv = row_vis<MASKED>(P, ri, q0, ctx - q_len);
    u32x4_t qop[KJ];
    load_q<D>(qop, P, q0, ri, kvh, g);
    // last key any row of this wave's tile sees (wave-uniform, -1 if no rows)
    const int wave_row0 = row0 + 16 * wave;
    const int wave_pmax =
        wave_row0 < rows_total ? ctx - q_len + min(wave_row0 + 15, rows_total - 1) / P.G : -1;
    // lowest key any row of the wave's tile, or of the workgroup, sees
    const int wave_lo = MASKED ? seq_lowest_key(P, ctx - q_len + wave_row0 / P.G) : 0;
    const int blk_lo = MASKED ? seq_lowest_key(P, ctx - q_len + row0 / P.G) : 0;

    // Staged parts sit PS bytes apart, PS = 128 modulo 256: the K tiles of a
    // step's two blocks then start 128 bytes apart modulo 256, so that the 16
    // lanes of one 256-byte LDS cycle that read both blocks hit distinct banks.
    constexpr int PS = (TB + 255) / 256 * 256 + 128;
    // NB step buffers, filled by asynchronous global-to-LDS copies that hold
    // no registers: the copies of NB - 1 steps are in flight while a step
    // computes.
    constexpr int NB = 4;
    __shared__ __attribute__((aligned(16))) uint8_t lds[NB][4 * PS];
    const size_t bstride = (size_t)P.Hkv * TB;
    const uint8_t *kbase = reinterpret_cast<const uint8_t *>(P.kp) + (size_t)kvh * TB;
    const uint8_t *vbase = reinterpret_cast<const uint8_t *>(P.vp) + (size_t)kvh * TB;
    const uint8_t *zero = reinterpret_cast<const uint8_t *>(g_zero_tile);
    const int nblk_seq = (ctx + kBlock - 1) / kBlock;
    // Wave w stages part w of every step: parts 0, 1 are the K tiles of the
    // step's blocks 0, 1; parts 2, 3 their V.
    const int blk = wave & 1;
    const bool is_v = wave >= 2;
    // LDS layout of the staged tiles: lds_k_piece, lds_v_piece (lane l of
    // copy v loads the piece that belongs at position l + 64 v). Each group
    // of 8 lanes writes 128 contiguous bytes, free of bank conflicts.

    // The block id of this wave's part of step c, through the scalar cache
    // (the step loop issues no vector loads of its own, so that its waits
    // count the copies alone); -1 past the sequence's blocks, whose parts
    // read the zero tile.
    const int32_t *bt_row = P.bt + (size_t)s * P.max_blocks_per_seq;
    const int jb_max = min(nblk_seq, P.max_blocks_per_seq);
    auto bid_of = [&](int c) {
        const int jb = 2 * c + blk;
        const int b = load_scalar(bt_row + min(jb, P.max_blocks_per_seq - 1));
        return (jb < jb_max && b >= 0 && b < P.num_blocks) ? b : -1;
    };
    // This wave's part of step c into buffer c % NB.
    auto stage = [&](int c, int b) {
        const uint8_t *src = b >= 0 ? (is_v ? vbase : kbase) + (size_t)b * bstride : zero;
        const uint32_t dst = lds_addr(&lds[c % NB][wave * PS]);
#pragma unroll
        for (int v = 0; v < NV; ++v)
            if (NP % 64 == 0 || lane + 64 * v < NP)
                lds_copy16(src,
                           (uint32_t)(is_v ? lds_v_piece<D, KF>(lane + 64 * v) : lds_k_piece<D, KF>(lane + 64 * v)) * 16,
                           dst + 1024 * v);
    };

    TileState<DT> spl, qtr, fin;  // quarter, split and row states of the wave's tile
    state_clear(spl);
    state_clear(qtr);
    state_clear(fin);
    const int nsteps = (p_max + kStep) / kStep;
    // Steps wholly below every row's lowest visible key change no state: the
    // walk starts at the step holding blk_lo.
    const int c_start = blk_lo > 0 ? blk_lo / kStep : 0;
    // The query rows (and visibility words) are in registers before the first
    // copy: a wait the compiler places for them inside the loop would count
    // the copies too, and drain them at every step.
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
#pragma unroll
    for (int c = c_start; c < c_start + NB - 1; ++c) stage(c, bid_of(c));
    int bid_next = bid_of(c_start + NB - 1);
    for (int c = c_start; c < nsteps; ++c) {
        const int kc = c * kStep;
        // This wave's copies of step c are done once at most those of the
        // NB - 2 steps after it are in flight; the barrier then shows every
        // wave's part, and that all waves are past step c - 1, whose buffer
        // the copy of step c + NB - 1 refills.
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"((NB - 2) * NV) : "memory");
        __syncthreads();
        stage(c + NB - 1, bid_next);
        bid_next = bid_of(c + NB);
        const uint8_t *buf = lds[c % NB];
        if (kc <= wave_pmax && (!MASKED || kc + kStep > wave_lo)) {
            Regs r;
            if constexpr (KF == kKvFp8)
                load_step8<D>(r, buf, buf + 2 * PS, buf + PS, buf + 3 * PS, g, n, [](int t) { return lds_k_pos(t); },
                              [](int row, int h) { return lds_v_half(row, h); });
            else if constexpr (KF == kKvFp4)
                load_step4<D, true>(r, buf, buf + 2 * PS, buf + PS, buf + 3 * PS, g, n);
            else
                load_step_lds<D>(r, reinterpret_cast<const uint16_t *>(buf), reinterpret_cast<const uint16_t *>(buf + 2 * PS),
                                 reinterpret_cast<const uint16_t *>(buf + PS),
                                 reinterpret_cast<const uint16_t *>(buf + 3 * PS), g, n);
            PoolT::mask(r, kc, ctx, g);
            // the first step of a quarter (quarter lengths divide every split start)
            const bool fresh = (kc & ((kc < kEdge ? kSplitA / 4 : kSplitB / 4) - 1)) == 0;
            PoolT::template update<MASKED, true>(qtr, r, qop, kc, rv, g, P.scale_log2, fresh);
        }
        // quarter and split boundaries fall on step boundaries; quarters are
        // kSplitA / 4 keys up to the edge and kSplitB / 4 after it, both
        // powers of two that divide every split start. Folded states are
        // emptied by their max alone: the accumulators of an empty quarter
        // are scaled by alpha = 0 in its first step with a key (the rescale is
        // unconditional here), and fold_state_flat weighs an empty state's
        // values by 0.
        const int next = kc + kStep;
        const int se = split_begin(split_index(kc) + 1);
        const int qmask = (next <= kEdge ? kSplitA / 4 : kSplitB / 4) - 1;
        const bool last = c + 1 == nsteps;
        if ((next & qmask) == 0 || last) {
            fold_state_flat(spl, qtr);
            qtr.m = -INFINITY;
            qtr.l = 0.f;
        }
        if (next == se || last) {
            fold_state_flat(fin, spl);
            spl.m = -INFINITY;
            spl.l = 0.f;
        }
    }
    // the copies past the last step land before the workgroup's LDS is released
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    f32x4_t o[DT];
    finalize(fin, sink_log2(P, kvh, ri.hl), o);
    store_out<DT>(P, q0, ri, kvh, g, o);
}

// ---------------------------------------------------------------------------
// fp32: one wave per (row, query head) over all its keys. Lane t takes key
// kc + t of each 64-key chunk for the score; lane d (and d + 64) owns channel
// d of the value sum.
// ---------------------------------------------------------------------------
__device__ inline int seq_of_row(const int32_t *qsl, int num_seqs, int row) {
    int lo = 0, hi = num_seqs;  // qsl[lo] <= row < qsl[hi]
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (qsl[mid] <= row) lo = mid; else hi = mid;
    }
    return lo;
}

template <int D>
__global__ __launch_bounds__(64) void attn_f32(AttnParams P) {
    constexpr int DU = D / 64;
    constexpr bool kPreV = D <= 64;  // a chunk's V rows of all four blocks held at once
    const int lane = threadIdx.x;
    const int i = blockIdx.x, h = blockIdx.y;
    // a decode batch's row i is sequence i
    const int s = P.decode_only ? i : seq_of_row(P.qsl, P.num_seqs, i);
    // block id of a key's block, read before the key is known to be in the
    // context (the index clamped to the table row; check() decides)
    auto bt_at = [&](int key) {
        return P.bt[(size_t)s * P.max_blocks_per_seq + min(key / kBlock, P.max_blocks_per_seq - 1)];
    };
    int raw = P.window == 0 ? bt_at(lane) : 0;  // the first chunk's, beside the context length
    const int q_len = P.decode_only ? 1 : P.qsl[s + 1] - P.qsl[s];
    const int ctx = P.ctx_lens[s];
    const int r = i - (P.decode_only ? i : P.qsl[s]);
    const int p = ctx - q_len + r;
    if (p < 0) return;
    const int kvh = h / P.G;
    // restricted visibility (tree window, sliding window)
    const int wbase = ctx - q_len;
    const int lo = P.window > 0 ? p - P.window + 1 : 0;
    const bool tree = P.tree_mask != nullptr;
    const uint32_t tm = tree ? P.tree_mask[i] | (1u << r) : 0xFFFFFFFFu;

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

    // the key's block, for every key up to p (lane 16 bb names block bb of
    // the chunk in the value pass, visible or not), else -1
    auto check = [&](int key, int b) {
        return (key <= p && key / kBlock < P.max_blocks_per_seq && b >= 0 && b < P.num_blocks) ? b : -1;
    };
    const int kc0 = lo > 0 ? lo / 64 * 64 : 0;
    if (P.window != 0) raw = bt_at(kc0 + lane);
    int phys = check(kc0 + lane, raw);
    for (int kc = kc0; kc <= p; kc += 64) {
        const int key = kc + lane;
        const bool vis = key <= p && key >= lo && (!tree || key < wbase || ((tm >> (key - wbase)) & 1u));
        // every read of the chunk first, with no branch between them: the
        // lane's key row, the V rows of the chunk's blocks (lane d: channel d)
        // and the next chunk's block ids. Keys and blocks outside the row read
        // block 0 (max(b, 0)), whose values the loop below never uses.
        const float *kb = kp + ((size_t)max(phys, 0) * P.Hkv + kvh) * tile;
        const int o = key % kBlock;
        f32x4_t kx[D / 4];
#pragma unroll
        for (int c = 0; c < D / 4; ++c) kx[c] = *reinterpret_cast<const f32x4_t *>(kb + (c * kBlock + o) * 4);
        float vv[kPreV ? 4 : 1][DU][kBlock];
        if constexpr (kPreV) {
#pragma unroll
            for (int bb = 0; bb < 4; ++bb) {
                const int pb = max(__builtin_amdgcn_readlane(phys, kBlock * bb), 0);
#pragma unroll
                for (int u = 0; u < DU; ++u) {
                    const float *vrow = vp + ((size_t)pb * P.Hkv + kvh) * tile + (size_t)(lane + 64 * u) * kBlock;
#pragma unroll
                    for (int q4 = 0; q4 < kBlock / 4; ++q4) {
                        const f32x4_t x = *reinterpret_cast<const f32x4_t *>(vrow + 4 * q4);
#pragma unroll
                        for (int e = 0; e < 4; ++e) vv[bb][u][4 * q4 + e] = x[e];
                    }
                }
            }
        }
        const int raw_next = kc + 64 <= p ? bt_at(kc + 64 + lane) : 0;
        float dot = 0.f;
        if (vis && phys >= 0) {
#pragma unroll
            for (int c = 0; c < D / 4; ++c) {
                dot = fmaf(qs[4 * c + 0], kx[c][0], dot);
                dot = fmaf(qs[4 * c + 1], kx[c][1], dot);
                dot = fmaf(qs[4 * c + 2], kx[c][2], dot);
                dot = fmaf(qs[4 * c + 3], kx[c][3], dot);
            }
        }
        const float sc = vis ? dot * P.scale_log2 : -INFINITY;
        float mx = sc;
#pragma unroll
        for (int o2 = 32; o2 >= 1; o2 >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o2, 64));
        if (mx != -INFINITY) {  // some key of the chunk visible (wave-uniform)
            const float m_new = fmaxf(m, mx);
            const float alpha = fast_exp2(m - m_new);
            const float pv = fast_exp2(sc - m_new);
            float rs = pv;
#pragma unroll
            for (int o2 = 32; o2 >= 1; o2 >>= 1) rs += __shfl_xor(rs, o2, 64);
            l = fmaf(alpha, l, rs);
            m = m_new;
#pragma unroll
            for (int u = 0; u < DU; ++u) acc[u] *= alpha;
#pragma unroll
            for (int bb = 0; bb < 4; ++bb) {
                const int kb0 = kc + kBlock * bb;
                if (kb0 > p) break;
                const int pb = __builtin_amdgcn_readlane(phys, kBlock * bb);
                if (pb < 0) continue;
#pragma unroll
                for (int u = 0; u < DU; ++u) {
                    float w8[kBlock];
                    if constexpr (kPreV) {
#pragma unroll
                        for (int tt = 0; tt < kBlock; ++tt) w8[tt] = vv[bb][u][tt];
                    } else {
                        const float *vrow =
                            vp + ((size_t)pb * P.Hkv + kvh) * tile + (size_t)(lane + 64 * u) * kBlock;
#pragma unroll
                        for (int q4 = 0; q4 < kBlock / 4; ++q4) {
                            const f32x4_t x = *reinterpret_cast<const f32x4_t *>(vrow + 4 * q4);
#pragma unroll
                            for (int e = 0; e < 4; ++e) w8[4 * q4 + e] = x[e];
                        }
                    }
#pragma unroll
                    for (int tt = 0; tt < kBlock; ++tt) {
                        const float w = bcast(pv, kBlock * bb + tt);
                        const float v = kb0 + tt <= p ? w8[tt] : 0.f;
                        acc[u] = fmaf(w, v, acc[u]);
                    }
                }
            }
        }
        phys = check(kc + 64 + lane, raw_next);
    }
    float lt = l;
    float al = 1.f;
    if (P.sinks) {
        const float sk = P.sinks[h] * kLog2e;
        const float M = fmaxf(m, sk);
        al = fast_exp2(m - M);
        lt = fmaf(l, al, fast_exp2(sk - M));
    }
#pragma unroll
    for (int u = 0; u < DU; ++u) P.out[((size_t)i * P.Hq + h) * D + lane + 64 * u] = (acc[u] * al) / lt;
}

// ---------------------------------------------------------------------------
// Scatter-write: one workgroup per 16 consecutive new tokens and one KV head.
// Every read is issued first: the tokens' slots, the group's K pieces in the
// tile's order (piece p is chunk p / 16 of token p % 16, so that a whole
// block goes out in contiguous 16-byte pieces) and its V rows row-major,
// which go to LDS before the one barrier. Where the 16 tokens fill one
// block in order (a prefill chunk, a verify window), the K tile and the
// transposed V tile are written as whole 16-byte pieces, the V columns
// gathered from LDS; otherwise each token's K chunks are 16-byte stores and
// its V values single-element stores.
// ---------------------------------------------------------------------------
template <typename T, int kMaxP>  // kMaxP: pieces per lane, 16 tokens x D / X pieces over 256 lanes
__global__ __launch_bounds__(256) void scatter_kernel(const T *__restrict__ kn, const T *__restrict__ vn,
                                                     const int32_t *__restrict__ slots, int n, T *kp, T *vp,
                                                     int num_blocks, int Hkv, int D) {
    constexpr int X = 16 / sizeof(T);  // elements per 16-byte piece
    const int tid = threadIdx.x, lane = tid & 63;
    const int i0 = blockIdx.x * kBlock, h = blockIdx.y;
    const int cpt = D / X;  // 16-byte pieces per token row
    const int np = kBlock * cpt;
    __shared__ int s_slot[kBlock];
    __shared__ __attribute__((aligned(16))) T sv[kBlock * 256];
    // indices clamped to the last token (n >= 1) and the last piece, so that
    // no read sits in a branch; the clamped tokens have no slot and the
    // clamped pieces are never stored
    const int slot_g = slots[min(i0 + (tid & (kBlock - 1)), n - 1)];
    u32x4_t kr[kMaxP], vr[kMaxP];
#pragma unroll
    for (int r = 0; r < kMaxP; ++r) {
        const int p = min(tid + 256 * r, np - 1);
        const int tk = p % kBlock, ck = p / kBlock;
        kr[r] = *reinterpret_cast<const u32x4_t *>(kn + ((size_t)min(i0 + tk, n - 1) * Hkv + h) * D + (size_t)ck * X);
        const int tv = p / cpt, cv = p - tv * cpt;
        vr[r] = *reinterpret_cast<const u32x4_t *>(vn + ((size_t)min(i0 + tv, n - 1) * Hkv + h) * D + (size_t)cv * X);
    }
#pragma unroll
    for (int r = 0; r < kMaxP; ++r) {
        const int p = tid + 256 * r;
        const int t = p / cpt, c = p - t * cpt;
        if (p < np) *reinterpret_cast<u32x4_t *>(sv + (size_t)t * D + (size_t)c * X) = vr[r];
    }
    if (tid < kBlock)
        s_slot[tid] = (i0 + tid < n && slot_g >= 0 && slot_g < num_blocks * kBlock) ? slot_g : -1;
    __syncthreads();
    // every wave tests the group itself: whole block, in order
    const int sl0 = s_slot[0];
    const int li = lane & (kBlock - 1);
    const bool full = __all(lane >= kBlock || (s_slot[li] >= 0 && s_slot[li] == sl0 + li && sl0 % kBlock == 0));
    if (full) {
        const size_t tile = ((size_t)(sl0 / kBlock) * Hkv + h) * D * kBlock;  // element offset
        // K: the tile [D/X][16][X] in order
#pragma unroll
        for (int r = 0; r < kMaxP; ++r) {
            const int p = tid + 256 * r;
            if (p < np) *reinterpret_cast<u32x4_t *>(kp + tile + (size_t)p * X) = kr[r];
        }
        // V [D][16]: each 16-byte piece of a channel row holds X tokens
        constexpr int PPR = kBlock / X;  // pieces per channel row
        for (int p = tid; p < D * PPR; p += 256) {
            const int ch = p / PPR, q = p % PPR;
            T e[X];
#pragma unroll
            for (int x = 0; x < X; ++x) e[x] = sv[(size_t)(q * X + x) * D + ch];
            u32x4_t w;
            __builtin_memcpy(&w, e, 16);
            *reinterpret_cast<u32x4_t *>(vp + tile + (size_t)ch * kBlock + q * X) = w;
        }
        return;
    }
#pragma unroll
    for (int r = 0; r < kMaxP; ++r) {
        const int p = tid + 256 * r;
        if (p >= np) continue;
        const int tk = p % kBlock, ck = p / kBlock;
        const int slk = s_slot[tk];
        if (slk >= 0) {
            const size_t tile = ((size_t)(slk / kBlock) * Hkv + h) * D * kBlock;
            *reinterpret_cast<u32x4_t *>(kp + tile + ((size_t)ck * kBlock + slk % kBlock) * X) = kr[r];
        }
        const int tv = p / cpt, cv = p - tv * cpt;
        const int slv = s_slot[tv];
        if (slv >= 0) {
            const size_t tile = ((size_t)(slv / kBlock) * Hkv + h) * D * kBlock;
            T e[X];
            __builtin_memcpy(e, &vr[r], 16);
#pragma unroll
            for (int x = 0; x < X; ++x) vp[tile + ((size_t)cv * X + x) * kBlock + slv % kBlock] = e[x];
        }
    }
}

// ---------------------------------------------------------------------------
// Scatter-write into 8-bit pools: one workgroup per 16 consecutive new tokens
// and one KV head; 16 lanes per token. Each (token, head) row is quantized:
// s = amax / 448, codes = E4M3 of x / s clamped to [-448, 448], rounded to
// nearest with ties to the even code by the conversion instruction (both
// divisions IEEE float32); a zero row stores s = 0 and zero codes. Codes and
// scales are then placed as in the tile layout: whole blocks written in order
// as 16-byte pieces gathered through LDS, other tokens piece by piece.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void scatter8_kernel(const uint16_t *__restrict__ kn, const uint16_t *__restrict__ vn,
                                                      const int32_t *__restrict__ slots, int n, uint8_t *kp,
                                                      uint8_t *vp, int num_blocks, int Hkv) {
    constexpr int TB = q8_tile_bytes<D>();
    constexpr int CPT = D / 16;  // channels per lane
    const int tid = threadIdx.x;
    const int i0 = blockIdx.x * kBlock, h = blockIdx.y;
    __shared__ int s_slot[kBlock];
    __shared__ __attribute__((aligned(16))) uint8_t kc[kBlock][D], vc[kBlock][D];
    __shared__ float ksc[kBlock], vsc[kBlock];
    // every read first, as vectors (indices clamped to the last token, n >= 1,
    // so that no read sits in a branch; clamped tokens are masked below)
    const int slot_g = slots[min(i0 + (tid & (kBlock - 1)), n - 1)];
    const int t = tid >> 4, part = tid & 15;  // token of the group, channel group
    const int i = i0 + t;
    const bool have = i < n;
    float xk[CPT], xv[CPT];
    {
        const size_t row = ((size_t)min(i, n - 1) * Hkv + h) * D + part * CPT;
        uint32_t wk[CPT / 2], wv[CPT / 2];
        if constexpr (CPT == 4) {
            const u32x2_t a = *reinterpret_cast<const u32x2_t *>(kn + row);
            const u32x2_t b = *reinterpret_cast<const u32x2_t *>(vn + row);
            wk[0] = a.x, wk[1] = a.y, wv[0] = b.x, wv[1] = b.y;
        } else {
            const u32x4_t a = *reinterpret_cast<const u32x4_t *>(kn + row);
            const u32x4_t b = *reinterpret_cast<const u32x4_t *>(vn + row);
            wk[0] = a.x, wk[1] = a.y, wk[2] = a.z, wk[3] = a.w;
            wv[0] = b.x, wv[1] = b.y, wv[2] = b.z, wv[3] = b.w;
        }
#pragma unroll
        for (int c = 0; c < CPT; ++c) {
            const uint32_t bk = c & 1 ? wk[c / 2] & 0xFFFF0000u : wk[c / 2] << 16;
            const uint32_t bv = c & 1 ? wv[c / 2] & 0xFFFF0000u : wv[c / 2] << 16;
            xk[c] = have ? __builtin_bit_cast(float, bk) : 0.f;
            xv[c] = have ? __builtin_bit_cast(float, bv) : 0.f;
        }
    }
    if (tid < kBlock)
        s_slot[tid] = (i0 + tid < n && slot_g >= 0 && slot_g < num_blocks * kBlock) ? slot_g : -1;
    auto quantize = [&](float (&x)[CPT], uint8_t *codes_row, float *scale_slot) {
        float amax = 0.f;
#pragma unroll
        for (int c = 0; c < CPT; ++c) amax = fmaxf(amax, fabsf(x[c]));
#pragma unroll
        for (int o = 8; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
        const float sc = __fdiv_rn(amax, 448.f);
        const float safe = sc > 0.f ? sc : 1.f;
#pragma unroll
        for (int c = 0; c < CPT; c += 2) {
            const float r0 = fminf(fmaxf(__fdiv_rn(x[c], safe), -448.f), 448.f);
            const float r1 = fminf(fmaxf(__fdiv_rn(x[c + 1], safe), -448.f), 448.f);
            const uint32_t w = sc > 0.f ? (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(r0, r1, 0, false) : 0u;
            codes_row[part * CPT + c] = (uint8_t)(w & 0xFF);
            codes_row[part * CPT + c + 1] = (uint8_t)((w >> 8) & 0xFF);
        }
        if (part == 0) *scale_slot = sc;
    };
    quantize(xk, kc[t], &ksc[t]);
    quantize(xv, vc[t], &vsc[t]);
    __syncthreads();
    // every wave tests the group itself: whole block, in order
    const int li = tid & (kBlock - 1);
    const bool s_full = __all((tid & 63) >= kBlock ||
                              (s_slot[li] >= 0 && s_slot[li] == s_slot[0] + li && s_slot[0] % kBlock == 0));
    // bytes of piece pc of a tile, from the group's codes (token tok of the
    // group sits at offset tok of the block in the whole-block case)
    auto k_piece = [&](int pc, int tok) {  // K piece ((p*4 + g)*16 + o): jj = 0 bytes then jj = 1 bytes
        const int q = pc >> 4, p = q >> 2, g = q & 3;
        uint8_t b[16];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            b[e] = kc[tok][64 * p + 8 * g + e];
            b[8 + e] = kc[tok][64 * p + 32 + 8 * g + e];
        }
        u32x4_t w;
        __builtin_memcpy(&w, b, 16);
        return w;
    };
    if (s_full) {
        const int blk = s_slot[0] / kBlock;
        uint8_t *kt = kp + ((size_t)blk * Hkv + h) * TB;
        uint8_t *vt = vp + ((size_t)blk * Hkv + h) * TB;
        for (int pc = tid; pc < D; pc += 256) {  // K code pieces: (p*4 + g)*16 + o
            *reinterpret_cast<u32x4_t *>(kt + (size_t)pc * 16) = k_piece(pc, pc & 15);
            // V piece ((d*16 + nn)*2 + hh): dd = 0 then dd = 1, tokens 8 hh + e
            const int row = pc >> 1, hh = pc & 1, d = row >> 4, nn = row & 15;
            uint8_t b[16];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                b[e] = vc[8 * hh + e][16 * (2 * d) + nn];
                b[8 + e] = vc[8 * hh + e][16 * (2 * d + 1) + nn];
            }
            u32x4_t w;
            __builtin_memcpy(&w, b, 16);
            *reinterpret_cast<u32x4_t *>(vt + (size_t)pc * 16) = w;
        }
        if (tid < kBlock) {
            reinterpret_cast<float *>(kt + 16 * D)[tid] = ksc[tid];
            reinterpret_cast<float *>(vt + 16 * D)[tid] = vsc[tid];
        }
        return;
    }
    const int sl = s_slot[t];
    if (!have || sl < 0) return;
    const int blk = sl / kBlock, o = sl % kBlock;
    uint8_t *kt = kp + ((size_t)blk * Hkv + h) * TB;
    uint8_t *vt = vp + ((size_t)blk * Hkv + h) * TB;
    // K: the token's D/8 runs of 8 codes (p, g, jj)
    for (int r = part; r < D / 8; r += 16) {
        const int p = r >> 3, g = (r >> 1) & 3, jj = r & 1;
        uint8_t b[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) b[e] = kc[t][64 * p + 32 * jj + 8 * g + e];
        u32x2_t w;
        __builtin_memcpy(&w, b, 8);
        *reinterpret_cast<u32x2_t *>(kt + ((size_t)((p * 4 + g) * kBlock + o)) * 16 + jj * 8) = w;
    }
    // V: one code per channel
#pragma unroll
    for (int c = part * CPT; c < part * CPT + CPT; ++c) {
        const int dt = c >> 4, nn = c & 15, d = dt >> 1, dd = dt & 1, hh = o >> 3, e = o & 7;
        vt[(((d * 16 + nn) * 2 + hh) * 2 + dd) * 8 + e] = vc[t][c];
    }
    if (part == 0) {
        reinterpret_cast<float *>(kt + 16 * D)[o] = ksc[t];
        reinterpret_cast<float *>(vt + 16 * D)[o] = vsc[t];
    }
}

// ---------------------------------------------------------------------------
// Scatter-write into 4-bit pools: the grid of scatter8_kernel. Each (token,
// head) row is quantized: s = amax / 6, codes = E2M1 of x / s clamped to
// [-6, 6], rounded to nearest with ties to the even code by the conversion
// instruction (both divisions IEEE float32); a zero row stores s = 0 and zero
// codes. A whole block written in order goes out as 16-byte pieces built in
// LDS. A token written alone owns its K run and its scales, but shares each
// V dword with the other tokens of its half block, which another workgroup
// may be writing at the same time: the group's tokens of one half block go
// in together, by a plain store where they fill the dword and otherwise by
// atomic nibble updates (clear, then set), which commute with the others'.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void scatter4_kernel(const uint16_t *__restrict__ kn, const uint16_t *__restrict__ vn,
                                                      const int32_t *__restrict__ slots, int n, uint8_t *kp,
                                                      uint8_t *vp, int num_blocks, int Hkv) {
    constexpr int TB = q4_tile_bytes<D>();
    constexpr int CPT = D / 16;  // channels per lane
    constexpr int KJ = D / 32, DT = D / 16;
    const int tid = threadIdx.x;
    const int i0 = blockIdx.x * kBlock, h = blockIdx.y;
    __shared__ __attribute__((aligned(16))) int s_slot[kBlock];
    __shared__ __attribute__((aligned(16))) uint8_t kc[kBlock][D], vc[kBlock][D];  // one code a byte
    __shared__ float ksc[kBlock], vsc[kBlock];
    // every read first, as vectors (indices clamped to the last token, n >= 1,
    // so that no read sits in a branch; clamped tokens are masked below)
    const int slot_g = slots[min(i0 + (tid & (kBlock - 1)), n - 1)];
    const int t = tid >> 4, part = tid & 15;  // token of the group, channel group
    const int i = i0 + t;
    const bool have = i < n;
    float xk[CPT], xv[CPT];
    {
        const size_t row = ((size_t)min(i, n - 1) * Hkv + h) * D + part * CPT;
        uint32_t wk[CPT / 2], wv[CPT / 2];
        if constexpr (CPT == 4) {
            const u32x2_t a = *reinterpret_cast<const u32x2_t *>(kn + row);
            const u32x2_t b = *reinterpret_cast<const u32x2_t *>(vn + row);
            wk[0] = a.x, wk[1] = a.y, wv[0] = b.x, wv[1] = b.y;
        } else {
            const u32x4_t a = *reinterpret_cast<const u32x4_t *>(kn + row);
            const u32x4_t b = *reinterpret_cast<const u32x4_t *>(vn + row);
            wk[0] = a.x, wk[1] = a.y, wk[2] = a.z, wk[3] = a.w;
            wv[0] = b.x, wv[1] = b.y, wv[2] = b.z, wv[3] = b.w;
        }
#pragma unroll
        for (int c = 0; c < CPT; ++c) {
            const uint32_t bk = c & 1 ? wk[c / 2] & 0xFFFF0000u : wk[c / 2] << 16;
            const uint32_t bv = c & 1 ? wv[c / 2] & 0xFFFF0000u : wv[c / 2] << 16;
            xk[c] = have ? __builtin_bit_cast(float, bk) : 0.f;
            xv[c] = have ? __builtin_bit_cast(float, bv) : 0.f;
        }
    }
    if (tid < kBlock)
        s_slot[tid] = (i0 + tid < n && slot_g >= 0 && slot_g < num_blocks * kBlock) ? slot_g : -1;
    auto quantize = [&](float (&x)[CPT], uint8_t *codes_row, float *scale_slot) {
        float amax = 0.f;
#pragma unroll
        for (int c = 0; c < CPT; ++c) amax = fmaxf(amax, fabsf(x[c]));
#pragma unroll
        for (int o = 8; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
        const float sc = __fdiv_rn(amax, 6.f);
        const float safe = sc > 0.f ? sc : 1.f;
#pragma unroll
        for (int c = 0; c < CPT; c += 2) {
            const float r0 = fminf(fmaxf(__fdiv_rn(x[c], safe), -6.f), 6.f);
            const float r1 = fminf(fmaxf(__fdiv_rn(x[c + 1], safe), -6.f), 6.f);
            const uint32_t w = sc > 0.f ? __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, r0, r1, 1.0f, 0) : 0u;
            codes_row[part * CPT + c] = (uint8_t)(w & 0xF);
            codes_row[part * CPT + c + 1] = (uint8_t)((w >> 4) & 0xF);
        }
        if (part == 0) *scale_slot = sc;
    };
    quantize(xk, kc[t], &ksc[t]);
    quantize(xv, vc[t], &vsc[t]);
    __syncthreads();
    // every wave tests the group itself: whole block, in order
    const int li = tid & (kBlock - 1);
    const bool s_full = __all((tid & 63) >= kBlock ||
                              (s_slot[li] >= 0 && s_slot[li] == s_slot[0] + li && s_slot[0] % kBlock == 0));
    // eight codes into a dword, the first in the low nibble
    auto pack8 = [](const uint8_t (&c)[8]) {
        uint32_t w = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) w |= (uint32_t)c[e] << (4 * e);
        return w;
    };
    if (s_full) {
        const int blk = s_slot[0] / kBlock;
        uint32_t *kt = reinterpret_cast<uint32_t *>(kp + ((size_t)blk * Hkv + h) * TB);
        uint32_t *vt = reinterpret_cast<uint32_t *>(vp + ((size_t)blk * Hkv + h) * TB);
        // 16-byte piece pc holds dwords 4 pc .. 4 pc + 3 of the code area
        for (int pc = tid; pc < D / 2; pc += 256) {
            u32x4_t wk, wv;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int w = 4 * pc + q;
                // K dword (g*16 + o) * KJ + j: token o, channels 32 j + 8 g + e
                const int j = w % KJ, go = w / KJ, g = go >> 4, o = go & 15;
                uint8_t ck[8], cv[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) ck[e] = kc[o][32 * j + 8 * g + e];
                // V dword (nn*2 + hh) * DT + dt: channel 16 dt + nn, tokens 8 hh + e
                const int dt = w % DT, nh = w / DT, nn = nh >> 1, hh = nh & 1;
#pragma unroll
                for (int e = 0; e < 8; ++e) cv[e] = vc[8 * hh + e][16 * dt + nn];
                wk[q] = pack8(ck);
                wv[q] = pack8(cv);
            }
            *reinterpret_cast<u32x4_t *>(kt + 4 * pc) = wk;
            *reinterpret_cast<u32x4_t *>(vt + 4 * pc) = wv;
        }
        if (tid < kBlock) {
            reinterpret_cast<float *>(kt + 2 * D)[tid] = ksc[tid];
            reinterpret_cast<float *>(vt + 2 * D)[tid] = vsc[tid];
        }
        return;
    }
    const int sl = s_slot[t];
    if (!have || sl < 0) return;
    // the group's tokens in this token's half block (slot / 8) and their
    // nibbles, from the 16 slots read at once
    uint32_t same = 0, nmask = 0;
    uint64_t nib = 0;  // 4 bits per token u: its nibble within the dword
    {
        int su[kBlock];
#pragma unroll
        for (int q = 0; q < kBlock / 4; ++q) {
            const int4 v = reinterpret_cast<const int4 *>(s_slot)[q];
            su[4 * q] = v.x, su[4 * q + 1] = v.y, su[4 * q + 2] = v.z, su[4 * q + 3] = v.w;
        }
#pragma unroll
        for (int u = 0; u < kBlock; ++u) {
            const bool m = (su[u] >> 3) == (sl >> 3);  // an empty slot (-1) never matches: sl >= 0
            same |= (uint32_t)m << u;
            nmask |= m ? 0xFu << (4 * (su[u] & 7)) : 0u;
            nib |= (uint64_t)(su[u] & 7) << (4 * u);
        }
    }
    const int blk = sl / kBlock, o = sl % kBlock;
    uint32_t *kt = reinterpret_cast<uint32_t *>(kp + ((size_t)blk * Hkv + h) * TB);
    uint32_t *vt = reinterpret_cast<uint32_t *>(vp + ((size_t)blk * Hkv + h) * TB);
    // K: the token's own runs, KJ dwords for each g
    for (int w = part; w < 4 * KJ; w += 16) {
        const int g = w / KJ, j = w % KJ;
        uint8_t ck[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) ck[e] = kc[t][32 * j + 8 * g + e];
        kt[(g * kBlock + o) * KJ + j] = pack8(ck);
    }
    // V: a dword holds one channel of a half block (8 tokens, nibble o & 7).
    // The group's tokens in one half block go in together, written by the
    // first of them: one plain store where they fill the dword, else one
    // atomic clear and one atomic set of their nibbles (which commute with
    // another group's updates of the other nibbles).
    const int hh = o >> 3;
    if (same == 1u << t) {  // alone in its half block here
        const int sh = 4 * (o & 7);
#pragma unroll
        for (int c = part * CPT; c < part * CPT + CPT; ++c) {
            const int dt = c >> 4, nn = c & 15;
            uint32_t *w = vt + (nn * 2 + hh) * DT + dt;
            atomicAnd(w, ~(0xFu << sh));
            atomicOr(w, (uint32_t)vc[t][c] << sh);
        }
    } else if (__builtin_ctz(same) == t) {
#pragma unroll
        for (int c = part * CPT; c < part * CPT + CPT; ++c) {
            const int dt = c >> 4, nn = c & 15;
            uint32_t val = (uint32_t)vc[t][c] << (4 * (o & 7));
            for (uint32_t m = same & (same - 1); m; m &= m - 1) {  // the others
                const int u = __builtin_ctz(m);
                val |= (uint32_t)vc[u][c] << (4 * (int)((nib >> (4 * u)) & 7));
            }
            uint32_t *w = vt + (nn * 2 + hh) * DT + dt;
            if (nmask == 0xFFFFFFFFu) {
                *w = val;
            } else {
                atomicAnd(w, ~nmask);
                atomicOr(w, val);
            }
        }
    }
    if (part == 0) {
        reinterpret_cast<float *>(kt + 2 * D)[o] = ksc[t];
        reinterpret_cast<float *>(vt + 2 * D)[o] = vsc[t];
    }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
// Workspace: the split maxima and sums, then the split accumulators.
struct WsLayout {
    size_t ml_bytes, acc_bytes;
    size_t total() const { return ml_bytes + acc_bytes; }
};

static size_t round256(size_t x) { return (x + 255) / 256 * 256; }

static WsLayout ws_layout(int64_t rows, int64_t Hq, int64_t D, int64_t splits) {
    const int64_t cells = rows * Hq * splits;
    WsLayout w;
    w.ml_bytes = round256((size_t)(cells * 8));
    w.acc_bytes = (size_t)(cells * D * 4);
    return w;
}

static bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
static bool aligned4(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

// A grid that leaves CUs free takes the two-stage variant: per-workgroup
// latency then decides the time, and occupancy does not matter.
template <int D, int NT>
static void launch_parallel(const AttnParams &P, hipStream_t st);

static int device_cus() {
    static int cache[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
    if (dev < 64 && cache[dev] > 0) return cache[dev];
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) cus = 1;
    if (dev < 64) cache[dev] = cus;
    return cus;
}

// workgroups of the parallel grid
static int64_t par_grid(const AttnParams &P) {
    if (P.pre_groups > 0)  // the slots of prefix_slot
        return (int64_t)P.Hkv * ((int64_t)P.pre_groups * P.pre_splits + P.pre_a +
                                 (int64_t)(P.num_seqs - P.pre_seqs) * P.max_splits);
    return (int64_t)P.Hkv * (P.seq_stride ? P.seq_stride : P.num_seqs) * P.grid_splits;
}

template <int D, int NT, bool APPEND, int KF, bool MASKED>
static void launch_parallel_as(const AttnParams &P, hipStream_t st) {
    const int64_t nwg = par_grid(P);
    // Two prefetch stages only on grids that leave CUs free. On grids that
    // queue, the one-stage variant keeps more workgroups resident: for 8- and
    // 4-bit tiles the conversions need the registers; for bf16 tiles the
    // extra slots measured 1 % faster on sink_decode's appending step and
    // even on its attention calls (whose fixed order had favoured two stages
    // by 3 % before the balanced order).
    if constexpr (NT == 1) {
        if (nwg <= device_cus()) {
            hipLaunchKernelGGL((attn_parallel<D, NT, true, APPEND, KF, MASKED>), dim3((unsigned)nwg), dim3(256), 0,
                               st, P);
            return;
        }
    }
    hipLaunchKernelGGL((attn_parallel<D, NT, false, APPEND, KF, MASKED>), dim3((unsigned)nwg), dim3(256), 0, st, P);
}

// The appending variant exists for single-tile rows only (forward_impl fuses
// no other batch).
template <int D, int NT, int KF, bool MASKED>
static void launch_parallel(const AttnParams &P, hipStream_t st) {
    if constexpr (KF != kKvBf16 || MASKED || NT != 1) launch_parallel_as<D, NT, false, KF, MASKED>(P, st);
    else if (P.k_new) launch_parallel_as<D, NT, true, kKvBf16, false>(P, st);
    else launch_parallel_as<D, NT, false, kKvBf16, false>(P, st);
}

template <int D, int NT>
static void launch_fold(const AttnParams &P, hipStream_t st) {
    const dim3 grid(P.num_seqs, P.Hkv, 16 * NT * D / 4 / 256);
    if (P.grid_splits > 16 && P.grid_splits <= 32)
        hipLaunchKernelGGL((attn_fold<D, NT, true>), grid, dim3(256), 0, st, P);
    else
        hipLaunchKernelGGL((attn_fold<D, NT, false>), grid, dim3(256), 0, st, P);
}

template <int D, int KF, bool MASKED>
static void launch_sequential(const AttnParams &P, int total_rows, hipStream_t st) {
    const int64_t items = ((int64_t)total_rows * P.G + kSeqRows - 1) / kSeqRows + P.num_seqs;
    hipLaunchKernelGGL((attn_sequential<D, KF, MASKED>), dim3((unsigned)(items * P.Hkv)), dim3(256), 0, st, P);
}

// The split and fold launches go to `st`; the sequential shape, when the
// batch has rows for it, to `seq_st`. When that is another stream it is
// launched first, so that its long row blocks are dispatched first.
template <int D, int KF, bool MASKED>
static void launch_mfma(const AttnParams &P, int max_q_len, int total_rows, hipStream_t st, hipStream_t seq_st) {
    const int rows_per_seq = max_q_len * P.G;
    const bool fold = P.max_splits > 1;
    if (rows_per_seq > kParRows && seq_st != st) launch_sequential<D, KF, MASKED>(P, total_rows, seq_st);
    if (P.G > kParRows) {
        // Every sequence brings at least G > 32 rows to its KV head: all of
        // them take the sequential shape, and the split and fold launches
        // would have nothing to do.
    } else if (rows_per_seq <= 16) {
        if (P.pre_groups > 0) {
            if constexpr (!MASKED)
                hipLaunchKernelGGL((attn_parallel<D, 1, false, false, KF, false, false, true>),
                                   dim3((unsigned)par_grid(P)), dim3(256), 0, st, P);
        } else {
            launch_parallel<D, 1, KF, MASKED>(P, st);
        }
        if (fold)
            launch_fold<D, 1>(P, st);
    } else {
        if (rows_per_seq > kParRows) {
            // A batch with prefill chunks: the one-tile instance, which holds
            // more waves per SIMD (measured on a mixed step: 14 % faster for
            // quantized tiles, 5 % for bf16; its two-stage variant was slower),
            // takes its decode rows, and sequences of 17 to 32 rows in two
            // passes, in one launch.
            if (P.pre_groups > 0) {
                if constexpr (!MASKED)
                    hipLaunchKernelGGL((attn_parallel<D, 1, false, false, KF, false, true, true>),
                                       dim3((unsigned)par_grid(P)), dim3(256), 0, st, P);
            } else {
                hipLaunchKernelGGL((attn_parallel<D, 1, false, false, KF, MASKED, true>),
                                   dim3((unsigned)par_grid(P)), dim3(256), 0, st, P);
            }
        } else {
            // two-tile windows take no prefix groups (a group tile holds
            // decode rows): their own grid
            AttnParams P2 = P;
            P2.pre_seqs = P2.pre_m = P2.pre_groups = P2.pre_splits = P2.pre_a = 0;
            launch_parallel<D, 2, KF, MASKED>(P2, st);
        }
        if (fold)
            launch_fold<D, 2>(P, st);
    }
    if (rows_per_seq > kParRows && seq_st == st) launch_sequential<D, KF, MASKED>(P, total_rows, st);
}

template <int D, int KF>
static void launch_mfma_vis(const AttnParams &P, int max_q_len, int total_rows, hipStream_t st,
                            hipStream_t seq_st) {
    if (P.tree_mask || P.window > 0) launch_mfma<D, KF, true>(P, max_q_len, total_rows, st, seq_st);
    else launch_mfma<D, KF, false>(P, max_q_len, total_rows, st, seq_st);
}

// A batch holding both prefill chunks and decode rows, captured into a
// graph, runs its two shapes on two streams: the sequential launch beside
// the split launch, which is bound by its dispatch and drain, not by the
// compute units the sequential shape keeps busy. The launches share no
// buffer: the sequential shape writes only its own rows' outputs, and the
// split and fold launches skip those rows. Each device has one side stream,
// at the default priority, forked from the caller's stream and joined back
// into it by two events; in the graph these become two edges. Eager calls
// keep both launches on the caller's stream: there the event pair costs
// more host and queue time than the overlap saves.
struct SideStream {
    hipStream_t s = nullptr;
    hipEvent_t fork = nullptr, join = nullptr;
    bool tried = false;
};
// Held from the fork's record to the join's, so that every wait sees the
// record of its own call.
static std::mutex g_side_mu;

// The side stream of the device `st` belongs to, created at the first call
// with both shapes on that device that is not under graph capture (a capture
// uses it, never creates it); nullptr where there is none (the sequential
// launch then stays on `st`). Called with g_side_mu held.
static const SideStream *side_stream(hipStream_t st) {
    static SideStream side[64];
    int dev = 0, cur = 0;
    if ((st ? hipStreamGetDevice(st, &dev) : hipGetDevice(&dev)) != hipSuccess || dev < 0 || dev >= 64)
        return nullptr;
    SideStream &x = side[dev];
    if (x.s || x.tried) return x.s ? &x : nullptr;
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(st, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone) return nullptr;
    if (hipGetDevice(&cur) != hipSuccess || (cur != dev && hipSetDevice(dev) != hipSuccess)) return nullptr;
    x.tried = true;  // a failed creation leaves this device on one stream
    hipStream_t sn = nullptr;
    hipEvent_t fk = nullptr, jn = nullptr;
    const bool s_ok = hipStreamCreateWithFlags(&sn, hipStreamNonBlocking) == hipSuccess;
    const bool f_ok = s_ok && hipEventCreateWithFlags(&fk, hipEventDisableTiming) == hipSuccess;
    const bool j_ok = f_ok && hipEventCreateWithFlags(&jn, hipEventDisableTiming) == hipSuccess;
    if (j_ok) {
        x.s = sn;
        x.fork = fk;
        x.join = jn;
    } else {  // release only what was created
        if (f_ok) (void)hipEventDestroy(fk);
        if (s_ok) (void)hipStreamDestroy(sn);
    }
    if (cur != dev) (void)hipSetDevice(cur);
    return x.s ? &x : nullptr;
}

}  // namespace pkv

extern "C" {

size_t paged_attention_workspace_size(int32_t num_seqs, int32_t total_q_rows, int32_t num_q_heads,
                                      int32_t head_dim, int32_t max_context_len) {
    if (num_seqs < 0 || total_q_rows < 0 || num_q_heads <= 0 || head_dim <= 0 || max_context_len < 0)
        return 0;
    return pkv::ws_layout(total_q_rows, num_q_heads, head_dim, pkv::num_splits(max_context_len)).total();
}

}  // extern "C"

namespace pkv {
// Split-state scratch of paged_attention_forward_noalloc, for callers that
// cannot allocate: 64 MiB, enough for 128 verify rows x 32 heads over 16384
// keys (40.5 MB). The module holds one copy per device for the process's
// life; calls on one device share it.
constexpr size_t kScratchBytes = size_t(64) << 20;
}  // namespace pkv

static __device__ __align__(256) unsigned char scratch[pkv::kScratchBytes];

namespace pkv {

// Device address of `scratch` on the device `hip_stream` belongs to (the
// current device for the null stream). In host code the array's name is a
// host-side stand-in, never a device address: the address comes from
// hipGetSymbolAddress, taken once per device with that device current.
static int scratch_on_stream(void *hip_stream, void **out) {
    static std::mutex mu;
    static void *addr[64] = {nullptr};
    int dev = 0;
    hipError_t e = hip_stream ? hipStreamGetDevice(reinterpret_cast<hipStream_t>(hip_stream), &dev)
                              : hipGetDevice(&dev);
    if (e != hipSuccess)
        PKV_FAIL(KV_EDEVICE, "paged_attention_forward_noalloc: no device for the stream: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= 64) PKV_FAIL(KV_EUNSUPPORTED, "paged_attention_forward_noalloc: device %d", dev);
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        int cur = 0;
        if ((e = hipGetDevice(&cur)) != hipSuccess)
            PKV_FAIL(KV_EDEVICE, "paged_attention_forward_noalloc: hipGetDevice: %s", hipGetErrorString(e));
        if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess)
            PKV_FAIL(KV_EDEVICE, "paged_attention_forward_noalloc: hipSetDevice(%d): %s", dev, hipGetErrorString(e));
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev) (void)hipSetDevice(cur);
        if (e != hipSuccess || !p)
            PKV_FAIL(KV_EDEVICE, "paged_attention_forward_noalloc: hipGetSymbolAddress(scratch) on device %d: %s",
                     dev, hipGetErrorString(e));
        addr[dev] = p;
    }
    *out = addr[dev];
    return KV_OK;
}

struct AppendArgs {
    const void *k_new, *v_new;
    const int32_t *slots;
};

struct MaskArgs {
    const uint32_t *tree_mask;
    int32_t window;
};

struct PrefixArgs {
    int32_t seqs, tokens;
};

static int forward_impl(const void *q, const void *k_pool, const void *v_pool, int32_t dtype,
                        const int32_t *block_tables, int32_t max_blocks_per_seq,
                        const int32_t *context_lens, const int32_t *query_start_loc, int32_t num_seqs,
                        int32_t total_q_rows, int32_t max_q_len, int32_t max_context_len, int32_t num_q_heads,
                        int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
                        float scale, const float *sinks, float *out, void *workspace, size_t workspace_bytes,
                        void *hip_stream, const AppendArgs *app, const MaskArgs *mk,
                        const PrefixArgs *pre = nullptr, bool may_fork = true) {
    if (dtype != KV_BF16 && dtype != KV_F32 && dtype != KV_FP8 && dtype != KV_FP4)
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
    if (num_q_heads > 65535)
        PKV_FAIL(KV_EINVAL, "paged_attention_forward: too many heads");
    if (!std::isfinite(scale)) PKV_FAIL(KV_EINVAL, "paged_attention_forward: scale is not finite");
    if (mk && mk->window < 0)
        PKV_FAIL(KV_EINVAL, "paged_attention_masked_forward: sliding_window %d < 0", mk->window);
    if (mk && mk->tree_mask && max_q_len > 32)
        PKV_FAIL(KV_EINVAL, "paged_attention_masked_forward: tree masks cover 32 window rows, max_q_len is %d",
                 max_q_len);
    if (pre && (pre->seqs < 0 || pre->tokens < 0))
        PKV_FAIL(KV_EINVAL, "paged_attention_prefix_forward: prefix_seqs %d and prefix_tokens %d must be >= 0",
                 pre->seqs, pre->tokens);
    if (mk && mk->tree_mask && !aligned4(mk->tree_mask))
        PKV_FAIL(KV_EINVAL, "paged_attention_masked_forward: tree_mask must be 4-byte aligned");
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
    if ((int64_t)num_kv_heads * (num_seqs + 3) * max_splits * 256 > (int64_t)UINT32_MAX)
        PKV_FAIL(KV_EINVAL, "paged_attention_forward: %d sequences x %d KV heads x %d splits exceed one launch",
                 num_seqs, num_kv_heads, max_splits);
    const WsLayout w = ws_layout(total_q_rows, num_q_heads, head_dim, max_splits);
    if (workspace_bytes < w.total())
        PKV_FAIL(KV_EINVAL, "paged_attention_forward: workspace of %zu bytes, need %zu", workspace_bytes,
                 w.total());

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
    P.decode_only = max_q_len == 1 && total_q_rows == num_seqs;
    // The dispatcher deals workgroups to the shader engines of a die in turn,
    // by count, not by work. A grid that queues takes the balanced order of
    // balanced_item where it applies; otherwise a sequence stride of 1 mod 4
    // (padding slots exit at once) moves each sequence to the next engine at
    // every split slot, so that no engine gets all the splits of the same
    // long sequences.
    // Under a sliding window, the keys some row of a sequence sees span at most
    // window + max_q_len - 1 positions, which meet at most that many keys / 256
    // (rounded up) + 1 splits.
    P.grid_splits = max_splits;
    if (mk && mk->window > 0)
        P.grid_splits = (int32_t)std::min<int64_t>(
            max_splits, ((int64_t)mk->window + max_q_len - 1 + kSplitA - 1) / kSplitA + 1);
    P.seq_stride = num_seqs;
    if ((int64_t)num_kv_heads * num_seqs * P.grid_splits > device_cus()) {
        // (measured: decode batches gain 2-5 %; batches with longer windows,
        // whose items are alike, lose up to 3 % to the extra round trip)
        const bool restricted = mk && (mk->tree_mask || mk->window > 0);
        if (P.decode_only && !restricted && num_seqs <= 64 && max_splits < 1024) P.seq_stride = 0;
        else P.seq_stride += (5 - num_seqs % 4) % 4;
    }
    // Shared prompt prefix: groups of up to four decode sequences (at most
    // 16 rows per group tile) over the splits wholly inside the prefix. The
    // fixed (not the balanced) slot order is then prefix_slot's.
    P.pre_seqs = P.pre_m = P.pre_groups = P.pre_splits = P.pre_a = 0;
    if (pre && pre->seqs > 1 && P.G <= 8) {
        const int seqs = std::min(pre->seqs, num_seqs);
        int js = 0;
        while (js < max_splits && split_begin(js + 1) <= pre->tokens) ++js;
        // the split holding the prefix's end joins the group items when the
        // prefix covers its first three quarters
        if (js > 0 && js < max_splits &&
            pre->tokens - split_begin(js) >= 3 * ((split_begin(js + 1) - split_begin(js)) / 4))
            ++js;
        if (js > 0) {
            P.pre_m = std::min(4, 16 / P.G);
            P.pre_seqs = seqs;
            P.pre_groups = (seqs + P.pre_m - 1) / P.pre_m;
            P.pre_splits = js;
            P.pre_a = seqs * (max_splits - js);
            P.seq_stride = num_seqs;
        }
    }
    P.scale_log2 = scale * kLog2e;
    P.k_new = P.v_new = nullptr;
    P.slots = nullptr;
    P.kp_w = P.vp_w = nullptr;
    P.tree_mask = mk ? mk->tree_mask : nullptr;
    P.window = mk ? mk->window : 0;
    hipStream_t st = reinterpret_cast<hipStream_t>(hip_stream);

    if (app) {
        // One new token per row, at the row's own position. A decode batch
        // whose rows fit one tile takes them inside the attention launch; any
        // other batch is scattered first, as two calls would.
        const bool fused = dtype == KV_BF16 && P.decode_only && max_q_len * P.G <= 16;
        if (fused) {
            P.k_new = static_cast<const uint16_t *>(app->k_new);
            P.v_new = static_cast<const uint16_t *>(app->v_new);
            P.slots = app->slots;
            P.kp_w = static_cast<uint16_t *>(const_cast<void *>(k_pool));
            P.vp_w = static_cast<uint16_t *>(const_cast<void *>(v_pool));
        } else {
            const int rc = kv_append_scatter(app->k_new, app->v_new, app->slots, total_q_rows,
                                             const_cast<void *>(k_pool), const_cast<void *>(v_pool), num_blocks,
                                             num_kv_heads, head_dim, block_size, dtype, hip_stream);
            if (rc != KV_OK) return rc;
        }
    }

    // both shapes in one batch, under graph capture: the sequential one on
    // the side stream
    std::unique_lock<std::mutex> side_lock(g_side_mu, std::defer_lock);
    const SideStream *sd = nullptr;
    hipStream_t seq_st = st;
    if (may_fork && dtype != KV_F32 && (int64_t)max_q_len * P.G > kParRows && P.G <= kParRows) {
        side_lock.lock();
        sd = side_stream(st);
        hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
        if (sd && hipStreamIsCapturing(st, &cs) == hipSuccess && cs == hipStreamCaptureStatusActive &&
            hipEventRecord(sd->fork, st) == hipSuccess && hipStreamWaitEvent(sd->s, sd->fork, 0) == hipSuccess) {
            seq_st = sd->s;
        } else {
            sd = nullptr;
            side_lock.unlock();
        }
    }
    (void)hipGetLastError();
    if (dtype == KV_BF16) {
        if (head_dim == 64) launch_mfma_vis<64, kKvBf16>(P, max_q_len, total_q_rows, st, seq_st);
        else launch_mfma_vis<128, kKvBf16>(P, max_q_len, total_q_rows, st, seq_st);
    } else if (dtype == KV_FP8) {
        if (head_dim == 64) launch_mfma_vis<64, kKvFp8>(P, max_q_len, total_q_rows, st, seq_st);
        else launch_mfma_vis<128, kKvFp8>(P, max_q_len, total_q_rows, st, seq_st);
    } else if (dtype == KV_FP4) {
        if (head_dim == 64) launch_mfma_vis<64, kKvFp4>(P, max_q_len, total_q_rows, st, seq_st);
        else launch_mfma_vis<128, kKvFp4>(P, max_q_len, total_q_rows, st, seq_st);
    } else {
        const dim3 grid(total_q_rows, num_q_heads);
        if (head_dim == 64) hipLaunchKernelGGL((attn_f32<64>), grid, dim3(64), 0, st, P);
        else hipLaunchKernelGGL((attn_f32<128>), grid, dim3(64), 0, st, P);
    }
    const hipError_t e = hipGetLastError();
    if (sd) {
        // the caller's stream waits for the side stream's launch
        hipError_t j = hipEventRecord(sd->join, sd->s);
        if (j == hipSuccess) j = hipStreamWaitEvent(st, sd->join, 0);
        if (j != hipSuccess)
            PKV_FAIL(KV_EDEVICE, "paged_attention_forward: joining the side stream failed: %s", hipGetErrorString(j));
    }
    if (e != hipSuccess)
        PKV_FAIL(KV_EDEVICE, "paged_attention_forward: launch failed: %s", hipGetErrorString(e));
    return KV_OK;
}

}  // namespace pkv

extern "C" {

int paged_attention_forward(const void *q, const void *k_pool, const void *v_pool, int32_t dtype,
                            const int32_t *block_tables, int32_t max_blocks_per_seq,
                            const int32_t *context_lens, const int32_t *query_start_loc,
                            int32_t num_seqs, int32_t total_q_rows, int32_t max_q_len,
                            int32_t max_context_len, int32_t num_q_heads, int32_t num_kv_heads,
                            int32_t head_dim, int32_t block_size, int32_t num_blocks, float scale,
                            const float *sinks, float *out, void *workspace, size_t workspace_bytes,
                            void *hip_stream) {
    return pkv::forward_impl(q, k_pool, v_pool, dtype, block_tables, max_blocks_per_seq, context_lens,
                             query_start_loc, num_seqs, total_q_rows, max_q_len, max_context_len, num_q_heads,
                             num_kv_heads, head_dim, block_size, num_blocks, scale, sinks, out, workspace,
                             workspace_bytes, hip_stream, nullptr, nullptr);
}

int paged_attention_forward_noalloc(const void *q, const void *k_pool, const void *v_pool, int32_t dtype,
                                    const int32_t *block_tables, int32_t max_blocks_per_seq,
                                    const int32_t *context_lens, const int32_t *query_start_loc,
                                    int32_t num_seqs, int32_t total_q_rows, int32_t max_q_len,
                                    int32_t max_context_len, int32_t num_q_heads, int32_t num_kv_heads,
                                    int32_t head_dim, int32_t block_size, int32_t num_blocks, float scale,
                                    const float *sinks, float *out, void *hip_stream) {
    if (num_q_heads <= 0 || head_dim <= 0 || num_seqs < 0 || total_q_rows < 0 || max_context_len < 0)
        PKV_FAIL(KV_EINVAL, "paged_attention_forward_noalloc: invalid sizes");
    const size_t need = paged_attention_workspace_size(num_seqs, total_q_rows, num_q_heads, head_dim,
                                                       max_context_len);
    if (need > pkv::kScratchBytes)
        PKV_FAIL(KV_EINVAL,
                 "paged_attention_forward_noalloc: this batch needs %zu bytes of split states, above the "
                 "library's fixed %zu-byte scratch array; call paged_attention_forward with a workspace",
                 need, pkv::kScratchBytes);
    void *ws = nullptr;
    const int rc = pkv::scratch_on_stream(hip_stream, &ws);
    if (rc != KV_OK) return rc;
    return pkv::forward_impl(q, k_pool, v_pool, dtype, block_tables, max_blocks_per_seq, context_lens,
                             query_start_loc, num_seqs, total_q_rows, max_q_len, max_context_len, num_q_heads,
                             num_kv_heads, head_dim, block_size, num_blocks, scale, sinks, out, ws,
                             pkv::kScratchBytes, hip_stream, nullptr, nullptr, nullptr, /*may_fork=*/false);
}

int paged_attention_prefix_forward(const void *q, const void *k_pool, const void *v_pool, int32_t dtype,
                                   const int32_t *block_tables, int32_t max_blocks_per_seq,
                                   const int32_t *context_lens, const int32_t *query_start_loc,
                                   int32_t num_seqs, int32_t total_q_rows, int32_t max_q_len,
                                   int32_t max_context_len, int32_t num_q_heads, int32_t num_kv_heads,
                                   int32_t head_dim, int32_t block_size, int32_t num_blocks, float scale,
                                   const float *sinks, int32_t prefix_seqs, int32_t prefix_tokens, float *out,
                                   void *workspace, size_t workspace_bytes, void *hip_stream) {
    const pkv::PrefixArgs pre{prefix_seqs, prefix_tokens};
    return pkv::forward_impl(q, k_pool, v_pool, dtype, block_tables, max_blocks_per_seq, context_lens,
                             query_start_loc, num_seqs, total_q_rows, max_q_len, max_context_len, num_q_heads,
                             num_kv_heads, head_dim, block_size, num_blocks, scale, sinks, out, workspace,
                             workspace_bytes, hip_stream, nullptr, nullptr, &pre);
}

int paged_attention_masked_forward(const void *q, const void *k_pool, const void *v_pool, int32_t dtype,
                                   const int32_t *block_tables, int32_t max_blocks_per_seq,
                                   const int32_t *context_lens, const int32_t *query_start_loc,
                                   int32_t num_seqs, int32_t total_q_rows, int32_t max_q_len,
                                   int32_t max_context_len, int32_t num_q_heads, int32_t num_kv_heads,
                                   int32_t head_dim, int32_t block_size, int32_t num_blocks, float scale,
                                   const float *sinks, const uint32_t *tree_mask, int32_t sliding_window,
                                   float *out, void *workspace, size_t workspace_bytes, void *hip_stream) {
    const pkv::MaskArgs mk{tree_mask, sliding_window};
    return pkv::forward_impl(q, k_pool, v_pool, dtype, block_tables, max_blocks_per_seq, context_lens,
                             query_start_loc, num_seqs, total_q_rows, max_q_len, max_context_len, num_q_heads,
                             num_kv_heads, head_dim, block_size, num_blocks, scale, sinks, out, workspace,
                             workspace_bytes, hip_stream, nullptr, &mk);
}

int paged_attention_append_forward(const void *q, const void *k_new, const void *v_new,
                                   const int32_t *slot_mapping, void *k_pool, void *v_pool, int32_t dtype,
                                   const int32_t *block_tables, int32_t max_blocks_per_seq,
                                   const int32_t *context_lens, const int32_t *query_start_loc,
                                   int32_t num_seqs, int32_t total_q_rows, int32_t max_q_len,
                                   int32_t max_context_len, int32_t num_q_heads, int32_t num_kv_heads,
                                   int32_t head_dim, int32_t block_size, int32_t num_blocks, float scale,
                                   const float *sinks, float *out, void *workspace, size_t workspace_bytes,
                                   void *hip_stream) {
    using namespace pkv;
    if (num_seqs > 0 && total_q_rows > 0) {
        if (!k_new || !v_new || !slot_mapping)
            PKV_FAIL(KV_EINVAL, "paged_attention_append_forward: k_new, v_new and slot_mapping are required");
        if (!aligned16(k_new) || !aligned16(v_new))
            PKV_FAIL(KV_EINVAL, "paged_attention_append_forward: k_new and v_new must be 16-byte aligned");
        if ((int64_t)num_blocks * kBlock > INT32_MAX)
            PKV_FAIL(KV_EINVAL, "paged_attention_append_forward: pool too large");
    }
    const AppendArgs app{k_new, v_new, slot_mapping};
    return forward_impl(q, k_pool, v_pool, dtype, block_tables, max_blocks_per_seq, context_lens, query_start_loc,
                        num_seqs, total_q_rows, max_q_len, max_context_len, num_q_heads, num_kv_heads, head_dim,
                        block_size, num_blocks, scale, sinks, out, workspace, workspace_bytes, hip_stream, &app,
                        nullptr);
}

int kv_append_scatter(const void *k_new, const void *v_new, const int32_t *slot_mapping, int32_t n,
                      void *k_pool, void *v_pool, int32_t num_blocks, int32_t num_kv_heads,
                      int32_t head_dim, int32_t block_size, int32_t dtype, void *hip_stream) {
    using namespace pkv;
    if (dtype != KV_BF16 && dtype != KV_F32 && dtype != KV_FP8 && dtype != KV_FP4)
        PKV_FAIL(KV_EUNSUPPORTED, "kv_append_scatter: dtype %d not supported", dtype);
    if ((dtype == KV_FP8 || dtype == KV_FP4) && head_dim != 64 && head_dim != 128)
        PKV_FAIL(KV_EUNSUPPORTED, "kv_append_scatter: 8- and 4-bit pools need head_dim 64 or 128, not %d", head_dim);
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
    const int64_t groups = ((int64_t)n + kBlock - 1) / kBlock;
    if (groups > INT32_MAX || num_kv_heads > 65535) PKV_FAIL(KV_EINVAL, "kv_append_scatter: too many tokens or heads");
    hipStream_t st = reinterpret_cast<hipStream_t>(hip_stream);
    (void)hipGetLastError();
    const dim3 grid((unsigned)groups, (unsigned)num_kv_heads);
    if (dtype == KV_FP4) {
        auto kn = static_cast<const uint16_t *>(k_new);
        auto vn = static_cast<const uint16_t *>(v_new);
        auto kpp = static_cast<uint8_t *>(k_pool);
        auto vpp = static_cast<uint8_t *>(v_pool);
        if (head_dim == 64)
            hipLaunchKernelGGL(scatter4_kernel<64>, grid, dim3(256), 0, st, kn, vn, slot_mapping, n, kpp, vpp, num_blocks,
                               num_kv_heads);
        else
            hipLaunchKernelGGL(scatter4_kernel<128>, grid, dim3(256), 0, st, kn, vn, slot_mapping, n, kpp, vpp,
                               num_blocks, num_kv_heads);
    } else if (dtype == KV_FP8) {
        auto kn = static_cast<const uint16_t *>(k_new);
        auto vn = static_cast<const uint16_t *>(v_new);
        auto kpp = static_cast<uint8_t *>(k_pool);
        auto vpp = static_cast<uint8_t *>(v_pool);
        if (head_dim == 64)
            hipLaunchKernelGGL(scatter8_kernel<64>, grid, dim3(256), 0, st, kn, vn, slot_mapping, n, kpp, vpp, num_blocks,
                               num_kv_heads);
        else
            hipLaunchKernelGGL(scatter8_kernel<128>, grid, dim3(256), 0, st, kn, vn, slot_mapping, n, kpp, vpp,
                               num_blocks, num_kv_heads);
    } else {
        // 16-byte pieces of a 16-token group over 256 lanes: 1, 2 or 4 per lane
        const int np = kBlock * head_dim * (dtype == KV_BF16 ? 2 : 4) / 16;
        auto launch = [&](auto kernel, auto *tag) {
            using T = std::remove_pointer_t<decltype(tag)>;
            hipLaunchKernelGGL(kernel, grid, dim3(256), 0, st, static_cast<const T *>(k_new),
                               static_cast<const T *>(v_new), slot_mapping, n, static_cast<T *>(k_pool),
                               static_cast<T *>(v_pool), num_blocks, num_kv_heads, head_dim);
        };
        if (dtype == KV_BF16) {
            uint16_t *tag = nullptr;
            if (np <= 256) launch(scatter_kernel<uint16_t, 1>, tag);
            else launch(scatter_kernel<uint16_t, 2>, tag);
        } else {
            float *tag = nullptr;
            if (np <= 256) launch(scatter_kernel<float, 1>, tag);
            else if (np <= 512) launch(scatter_kernel<float, 2>, tag);
            else launch(scatter_kernel<float, 4>, tag);
        }
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) PKV_FAIL(KV_EDEVICE, "kv_append_scatter: launch failed: %s", hipGetErrorString(e));
    return KV_OK;
}

}  // extern "C"
