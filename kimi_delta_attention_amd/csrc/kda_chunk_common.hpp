// kda_chunk_common.hpp -- pieces shared by the chunked forward and backward
// kernels: chunk geometry, MFMA tile helpers and the workspace layout.
//
// Chunk size is fixed at 64 tokens; inside a chunk rows are grouped in four
// 16-row sub-blocks (the MFMA tile height).
#pragma once

#include "kda_device.hpp"
#include "kda_launch.hpp"

#include <type_traits>

namespace kda {

constexpr int kChunk = 64;
constexpr int kSub = 16;
constexpr int kThreads = 256;
// Grid of the kernels that loop over (chunk, head) slots: one workgroup per
// compute unit of an MI355X (their LDS use allows one per CU).
constexpr int kPersistentGrid = 256;
// Diagonal 16-row sub-blocks whose accumulated decay span stays under this
// bound are factorised through the row before the block (factors up to
// e^kSpanLimit, finite in fp32); wider spans go through the level
// decomposition below, whose factors are all at most 1.
constexpr float kSpanLimit = 85.0f;

typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));
typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- MFMA tiles
// C[16x16] += A[16 x KS] * B[KS x 16] with both operands stored k-contiguous
// in LDS: A as [m][k], B transposed as [n][k].  Lane l supplies row l%16 and
// the k-slice (l/16)*KPL .. +KPL; the accumulator holds column l%16, rows
// 4*(l/16) .. +3.
template <bool BF> struct Mma;

template <> struct Mma<true> {        // bf16 inputs, fp32 accumulate
    using ET = uint16_t;              // LDS / workspace element (bf16 bits)
    static constexpr int KS = 32;
    static constexpr int KPL = 8;
    static constexpr int PAD = 8;     // row padding (elements) against bank conflicts
    using Frag = bf16x8;
    __device__ __forceinline__ static Frag load(const ET* base, int ld, int r0, int k0, int lane) {
        return *reinterpret_cast<const Frag*>(base + (r0 + (lane & 15)) * ld + k0 + (lane >> 4) * 8);
    }
    __device__ __forceinline__ static f32x4 mma(Frag a, Frag b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
    // Fragment times 8 per-k factors (fp32), rounded back to bf16.
    __device__ __forceinline__ static Frag scale(Frag f, const float* s) {
        u16x8 u = __builtin_bit_cast(u16x8, f);
        u16x8 r;
#pragma unroll
        for (int j = 0; j < 8; ++j) r[j] = f32_to_bf16_bits(bf16_bits_to_f32(u[j]) * s[j]);
        return __builtin_bit_cast(Frag, r);
    }
    __device__ __forceinline__ static ET from_f32(float x) { return f32_to_bf16_bits(x); }
    __device__ __forceinline__ static float to_f32(ET x) { return bf16_bits_to_f32(x); }
    // KPL fp32 values rounded into one fragment
    __device__ __forceinline__ static Frag pack(const float (&x)[KPL]) {
        u16x8 u;
#pragma unroll
        for (int e = 0; e < 8; ++e) u[e] = f32_to_bf16_bits(x[e]);
        return __builtin_bit_cast(Frag, u);
    }
};

template <> struct Mma<false> {       // fp32 inputs, fp32 accumulate
    using ET = float;
    static constexpr int KS = 4;
    static constexpr int KPL = 1;
    static constexpr int PAD = 4;     // keeps rows 16-byte aligned and conflict-free
    using Frag = float;
    __device__ __forceinline__ static Frag load(const ET* base, int ld, int r0, int k0, int lane) {
        return base[(r0 + (lane & 15)) * ld + k0 + (lane >> 4)];
    }
    __device__ __forceinline__ static f32x4 mma(Frag a, Frag b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
    }
    __device__ __forceinline__ static Frag scale(Frag f, const float* s) { return f * s[0]; }
    __device__ __forceinline__ static ET from_f32(float x) { return x; }
    __device__ __forceinline__ static float to_f32(ET x) { return x; }
    __device__ __forceinline__ static Frag pack(const float (&x)[KPL]) { return x[0]; }
};

// ---- level decomposition of a diagonal 16-row sub-block
// The score X_ij = sum_c x_ic k_jc e^(G_ic - G_jc) of a row pair (i, j), j < i,
// inside one 16-row sub-block is factorised through a reference row that lies
// between them, so that both factors are at most 1 for any decay span: with
// positions a = i mod 16 and b = j mod 16, the pair belongs to level h, the
// highest bit in which a and b differ (h in {8, 4, 2, 1}); i lies in the later
// half (bit h set) and j in the earlier half of the same 2h-row group, and the
// reference is that group's row (a & ~(2h - 1)) + h - 1, the last row of the
// earlier half.  Each level is one product with the rows of the later half as
// left operand (factor e^(G_i - G_ref)) and the rows of the earlier half as
// right operand (factor e^(G_ref - G_j)); the diagonal i = j carries no decay.

// Factor of row position pos at level h: e^(G_pos - G_ref) in the later half,
// e^(G_ref - G_pos) in the earlier half.
__device__ __forceinline__ float level_fac(int pos, int h, float g_pos, float g_ref) {
    return (pos & h) ? __expf(g_pos - g_ref) : __expf(g_ref - g_pos);
}

// True when (a, b) is a pair of level h with a in the later half.
__device__ __forceinline__ bool level_pair(int a, int b, int h) {
    return (a & h) && !(b & h) && ((a ^ b) < 2 * h);
}

// 4-bit mask over the positions base .. base + 3 of the other index: with
// row_is_later, bit e is level_pair(pos, base + e, h) (pos the later row), else
// level_pair(base + e, pos, h) (pos the earlier row).
__device__ __forceinline__ unsigned level_keep(int pos, int base, int h, bool row_is_later) {
    unsigned m = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e)
        if (row_is_later ? level_pair(pos, base + e, h) : level_pair(base + e, pos, h)) m |= 1u << e;
    return m;
}

// ---------------------------------------------------------------- geometry
// Sequence bounds: dense input (cu == nullptr) or packed offsets.  Offsets are
// clamped into [0, T_total] so malformed device data cannot move an access
// outside the tensors.
__device__ __forceinline__ void seq_bounds(const ChunkParams& p, int n, int64_t& start, int& len) {
    if (p.cu_seqlens) {
        const int64_t total = static_cast<int64_t>(p.T);
        int64_t a = p.cu_seqlens[n], b = p.cu_seqlens[n + 1];
        a = a < 0 ? 0 : (a > total ? total : a);
        b = b < a ? a : (b > total ? total : b);
        start = a;
        len = static_cast<int>(b - a);
    } else {
        start = static_cast<int64_t>(n) * p.T;
        len = p.T;
    }
}

__device__ __forceinline__ int n_chunks(int len) { return (len + kChunk - 1) / kChunk; }

// Workspace layout of the per-chunk operands produced by the prep kernel, per
// (chunk, head) slot, all [row][col] with the column fastest:
//   QE  [64][K]  scale * q^ * exp(G)                     (ET)
//   W   [64][K]  T diag(beta) (k^ * exp(G))              (ET)
//   KD  [64][K]  k^ * exp(G_last - G)                    (ET)
//   U   [64][V]  T diag(beta) v                          (ET)
//   TB  [64][64] T diag(beta), T = (I + A)^-1            (ET)
//   MS  [64][64] scale * tril(q^ k^T decayed)            (ET)
//   GC  [K]      exp(G_last)                             (fp32)
// G is the inclusive cumulative log-decay inside the chunk.  With S the state
// entering the chunk, D = U - W S, O = QE S + MS D and S' = GC * S + KD^T D.
template <int K, bool BF, int V = K>
struct PrepLayout {
    using ET = typename Mma<BF>::ET;
    static constexpr size_t kQE = 0;
    static constexpr size_t kW = kQE + sizeof(ET) * kChunk * K;
    static constexpr size_t kKD = kW + sizeof(ET) * kChunk * K;
    static constexpr size_t kU = kKD + sizeof(ET) * kChunk * K;
    static constexpr size_t kTB = kU + sizeof(ET) * kChunk * V;
    static constexpr size_t kMS = kTB + sizeof(ET) * kChunk * kChunk;
    static constexpr size_t kGC = kMS + sizeof(ET) * kChunk * kChunk;
    static constexpr size_t kBytes = ((kGC + sizeof(float) * K) + 255) / 256 * 256;
};

// Backward-only additions to a slot, placed after the PrepLayout operands:
//   KE   [64][K]  k^ * exp(G)                     (ET)
//   T    [64][64] (I + A)^-1                      (ET)
//   AK   [64][64] strict_tril(k^ k^T decayed)      (ET)
//   S    [V][K]   state entering the chunk, transposed          (ET)
//   DS   [V][K]   gradient of the state leaving it, transposed (ET)
//   DQE, DKE, DKD [64][K]  gradients of the QE, KE, KD operands, summed over V (ET)
//   DMS, DTB      [64][64] gradients of MS and TB, summed over V (ET)
//   DGAM [K]      gradient of exp(G_last) (fp32)
//   GP   [K + 1]  this chunk's share of d(dt_bias) and d(A_log) (fp32)
template <int K, bool BF, int V = K>
struct BwdExtra {
    using ET = typename Mma<BF>::ET;
    static constexpr size_t kKE = PrepLayout<K, BF, V>::kBytes;
    static constexpr size_t kT = kKE + sizeof(ET) * kChunk * K;
    static constexpr size_t kAK = kT + sizeof(ET) * kChunk * kChunk;
    static constexpr size_t kS = kAK + sizeof(ET) * kChunk * kChunk;
    static constexpr size_t kDS = kS + sizeof(ET) * K * V;
    static constexpr size_t kDQE = kDS + sizeof(ET) * K * V;
    static constexpr size_t kDKE = kDQE + sizeof(ET) * kChunk * K;
    static constexpr size_t kDKD = kDKE + sizeof(ET) * kChunk * K;
    static constexpr size_t kDMS = kDKD + sizeof(ET) * kChunk * K;
    static constexpr size_t kDTB = kDMS + sizeof(ET) * kChunk * kChunk;
    static constexpr size_t kDGAM = kDTB + sizeof(ET) * kChunk * kChunk;
    static constexpr size_t kGP = kDGAM + sizeof(float) * K;
    static constexpr size_t kBytes = ((kGP + sizeof(float) * (K + 1)) + 255) / 256 * 256;
};

__host__ __device__ inline size_t align256(size_t x) { return (x + 255) / 256 * 256; }

// The plan at the head of the workspace (packed input only):
//   chunk_off [N + 1]  int32, chunk_off[n] = chunks of sequences 0..n-1;
//   slot map  [bound]  int4 {n, j, start, len} per chunk slot (256-byte
//                      aligned), n = -1 for slots past the last chunk,
// written by plan_chunks_kernel, so that a parallel kernel locates its slot
// with one 16-byte load instead of a search over chunk_off and cu_seqlens.
__host__ __device__ inline size_t plan_map_offset(int N) {
    return align256(sizeof(int32_t) * (static_cast<size_t>(N) + 1));
}

__host__ inline size_t chunk_off_bytes(const ChunkParams& p) {
    size_t b = plan_map_offset(p.N);
    if (p.cu_seqlens) b += align256(sizeof(int32_t) * 4 * static_cast<size_t>(p.total_chunks_bound));
    return b;
}

// Chunk slot of chunk j of sequence n (slots are numbered over all sequences).
__device__ __forceinline__ int64_t chunk_slot(const ChunkParams& p, const int32_t* chunk_off, int n,
                                              int j) {
    const int64_t base = p.cu_seqlens ? chunk_off[n] : static_cast<int64_t>(n) * n_chunks(p.T);
    return base + j;
}

// Chunks of sequence n that the state passes walk.  For packed offsets that
// break the non-decreasing rule the clamped lengths can add up to more chunks
// than there are slots; a chain then stops at the last slot, so that every
// workspace access stays inside it (the results are unspecified).
__device__ __forceinline__ int chain_chunks(const ChunkParams& p, const int32_t* chunk_off, int n, int len) {
    const int nc = n_chunks(len);
    if (!p.cu_seqlens) return nc;
    const int room = p.total_chunks_bound - chunk_off[n];
    return nc < room ? nc : (room > 0 ? room : 0);
}

// Slot c -> (sequence n, chunk j, sequence start row, sequence length);
// false when c is past the last chunk.
__device__ __forceinline__ bool slot_locate(const ChunkParams& p, const int32_t* chunk_off, int c, int& n, int& j,
                                            int64_t& start, int& len) {
    if (!p.cu_seqlens) {
        const int nc = n_chunks(p.T);
        if (nc == 0) return false;
        n = c / nc;
        j = c % nc;
        start = static_cast<int64_t>(n) * p.T;
        len = p.T;
        return n < p.N;
    }
    const int4 e = reinterpret_cast<const int4*>(reinterpret_cast<const uint8_t*>(chunk_off) +
                                                 plan_map_offset(p.N))[c];
    n = e.x;
    j = e.y;
    start = e.z;
    len = e.w;
    return n >= 0;
}

// Column-block grid remap: all V-column blocks of one (sequence, head) chain
// get block ids with the same residue mod 8, i.e. land on the same XCD and
// share its L2 for the chain's per-chunk operands.
__device__ __forceinline__ bool chain_of_block(int bid, int n_chains, int nvb, int& chain, int& vb) {
    const int grp = bid / (8 * nvb);
    const int rem = bid % (8 * nvb);
    vb = rem / 8;
    chain = grp * 8 + rem % 8;
    return chain < n_chains;
}

// Head of item `item` (item = slot * H + position among the slot's heads) in
// the persistent loops over (slot, head) items.  With rotate, the heads of a
// slot are rotated by slot / max(1, grid / H), so that a workgroup walking
// items b, b + grid, b + 2 grid, ... meets a different head at each step
// rather than one head throughout: with the in-kernel gates the work per slot
// differs several-fold between fast- and slow-decaying heads (the level paths
// of over-wide sub-blocks), and a fixed head per workgroup leaves the kernel
// waiting on the workgroups of the fast heads.  A bijection on the heads of
// each slot, so every (slot, head) is still taken exactly once.  Without
// rotate (the log-decay gate, uniform work), the plain order measured slightly
// faster.
__host__ __device__ __forceinline__ int item_head(int64_t item, int H, int64_t grid, bool rotate) {
    if (!rotate) return static_cast<int>(item % H);
    const int64_t c = grid / H > 1 ? grid / H : 1;
    return static_cast<int>((item % H + (item / H) / c) % H);
}

__host__ __device__ constexpr int chain_grid(int n_chains, int nvb) {
    return ((n_chains + 7) / 8) * 8 * nvb;
}

}  // namespace kda
