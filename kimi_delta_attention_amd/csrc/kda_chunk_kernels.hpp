// kda_chunk_kernels.hpp -- the per-chunk preparation kernel and the forward
// state-pass kernel, shared by the forward and the backward translation units.
//
// The chunk form computes exactly the token recurrence of the
// "atlas_core/kimi_k3/kda.rs" page (module doc "Recurrence"): per chunk of 64
// rows, with G the inclusive cumulative log-decay inside the chunk,
//   A  = diag(beta) * strict_tril(sum_c k_i k_j exp(G_i - G_j))
//   M  = tril(sum_c q_i k_j exp(G_i - G_j))            (diagonal included)
//   T  = (I + A)^-1                                     (the inverse named in the
//                                                        "K3/kda/ops/api.py" page's
//                                                        l2-norm warning)
//   D  = T diag(beta) (v - (k exp(G)) S)
//   O  = scale * ((q exp(G)) S + M D)
//   S' = diag(exp(G_last)) S + (k exp(G_last - G))^T D
// The in-kernel prologue (q/k L2 norm, beta sigmoid, gate transform) follows
// the order of api.py chunk_kda; the gate fused with its cumulative sum is the
// in-kernel gate path of the "KDA <=> FLA Parity in Primus" page (section
// "What changed and why", table A).
//
//   prep   one workgroup per (chunk, head), fully parallel: prologue, cumsum,
//          the exponentials, A and M on MFMA, the blocked triangular inverse;
//          writes the chunk's operands (PrepLayout) to its workspace slot.
//   state  one workgroup per (sequence, head, V-column block), sequential over
//          the sequence's chunks: four small MFMA products per chunk with the
//          fp32 state held in MFMA accumulators.  Every term is local to a
//          value column, so column blocks of one head are independent.
//
// Overflow-safe decay: exponents are always taken against a reference row so
// that no factor exceeds 1, except on the diagonal 16x16 sub-blocks, where the
// reference is the row before the block and the opposite factor is at most
// exp(span of the block).  A block whose span exceeds kSpanLimit for any
// channel (possible only with unbounded gates) is formed by the level
// decomposition instead (kda_chunk_common.hpp): four more products, each with
// a reference row between the rows it pairs, so every factor is at most 1.
#pragma once

#include "kda_chunk_common.hpp"
#include "kda_lds.hpp"

namespace kda {

// ------------------------------------------------------------------ plan
// The plan of a packed call (layout at plan_map_offset): chunk_off by a
// block-wide scan of the sequences' chunk counts (kPlanThreads per round:
// shuffle scans within each wave, then the waves' totals), then the slot map,
// each slot's sequence found by a binary search over the offsets (read from
// LDS up to kPlanLdsSeqs sequences, from chunk_off beyond).  One workgroup of
// kPlanThreads; sequence offsets are clamped into [0, T] as in seq_bounds.
constexpr int kPlanThreads = 1024;
constexpr int kPlanLdsSeqs = 4096;
static __global__ __launch_bounds__(kPlanThreads) void plan_chunks_kernel(const int32_t* cu, int N, int T,
                                                                          int32_t* chunk_off, int bound) {
    constexpr int NW = kPlanThreads / 64;
    __shared__ int wsum[NW];
    __shared__ int offs[kPlanLdsSeqs + 1];
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    auto clamp_seq = [&](int n, int& a, int& b) {
        a = cu[n];
        b = cu[n + 1];
        a = a < 0 ? 0 : (a > T ? T : a);
        b = b < a ? a : (b > T ? T : b);
    };
    int carry = 0;
    for (int base = 0; base < N; base += kPlanThreads) {
        const int n = base + t;
        int c = 0;
        if (n < N) {
            int a, b;
            clamp_seq(n, a, b);
            c = n_chunks(b - a);
        }
        int v = c;  // inclusive scan within the wave
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int u = __shfl_up(v, o, 64);
            if (lane >= o) v += u;
        }
        if (lane == 63) wsum[w] = v;
        __syncthreads();
        int before = 0, total = 0;
#pragma unroll
        for (int q = 0; q < NW; ++q) {
            const int s_ = wsum[q];
            if (q < w) before += s_;
            total += s_;
        }
        if (n < N) {
            const int off = carry + before + v - c;
            chunk_off[n] = off;
            if (n < kPlanLdsSeqs) offs[n] = off;
        }
        carry += total;
        __syncthreads();  // wsum is rewritten by the next round
    }
    if (t == 0) {
        chunk_off[N] = carry;
        if (N <= kPlanLdsSeqs) offs[N] = carry;
    }
    __syncthreads();  // the offsets are read back below by other threads of this workgroup
    const bool in_lds = N <= kPlanLdsSeqs;
    auto off_at = [&](int m) { return in_lds ? offs[m] : chunk_off[m]; };
    int4* map = reinterpret_cast<int4*>(reinterpret_cast<uint8_t*>(chunk_off) + plan_map_offset(N));
    for (int c = t; c < bound; c += kPlanThreads) {
        int4 e = {-1, 0, 0, 0};
        if (c < carry) {
            int lo = 0, hi = N - 1;  // last n with chunk_off[n] <= c
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (off_at(mid) <= c) lo = mid; else hi = mid - 1;
            }
            int a, b;
            clamp_seq(lo, a, b);
            e = int4{lo, c - off_at(lo), a, b - a};
        }
        map[c] = e;
    }
}

// Vector load of CPT consecutive elements into fp32 registers.
template <int CPT>
__device__ __forceinline__ void load_row(const uint16_t* src, float* dst) {
    static_assert(CPT % 8 == 0, "bf16 rows are loaded 8 at a time");
#pragma unroll
    for (int v = 0; v < CPT / 8; ++v) {
        const u16x8 u = *reinterpret_cast<const u16x8*>(src + 8 * v);
#pragma unroll
        for (int e = 0; e < 8; ++e) dst[8 * v + e] = bf16_bits_to_f32(u[e]);
    }
}
template <int CPT>
__device__ __forceinline__ void load_row(const float* src, float* dst) {
    static_assert(CPT % 4 == 0, "fp32 rows are loaded 4 at a time");
#pragma unroll
    for (int v = 0; v < CPT / 4; ++v) {
        const f32x4 u = *reinterpret_cast<const f32x4*>(src + 4 * v);
#pragma unroll
        for (int e = 0; e < 4; ++e) dst[4 * v + e] = u[e];
    }
}
template <int CPT>
__device__ __forceinline__ void store_row(uint16_t* dst, const float* src) {
#pragma unroll
    for (int v = 0; v < CPT / 8; ++v) {
        u16x8 u;
#pragma unroll
        for (int e = 0; e < 8; ++e) u[e] = f32_to_bf16_bits(src[8 * v + e]);
        *reinterpret_cast<u16x8*>(dst + 8 * v) = u;
    }
}
template <int CPT>
__device__ __forceinline__ void store_row(float* dst, const float* src) {
#pragma unroll
    for (int v = 0; v < CPT / 4; ++v) {
        f32x4 u = {src[4 * v], src[4 * v + 1], src[4 * v + 2], src[4 * v + 3]};
        *reinterpret_cast<f32x4*>(dst + 4 * v) = u;
    }
}

// Accumulator tile (16 x 16) store helpers.  Lane l holds column l % 16 and
// rows 4 (l / 16) .. +3 of the tile at (r0, c0).
template <class MM>
__device__ __forceinline__ void tile_store(typename MM::ET* dst, int ld, int r0, int c0, f32x4 v, int lane) {
#pragma unroll
    for (int r = 0; r < 4; ++r) dst[(r0 + 4 * (lane >> 4) + r) * ld + c0 + (lane & 15)] = MM::from_f32(v[r]);
}
// Transposed: the lane's four rows are consecutive in dst, written as one
// 8-byte (bf16) or 16-byte (fp32) store; ld and r0 keep it aligned.
template <class MM>
__device__ __forceinline__ void tile_store_t(typename MM::ET* dst, int ld, int r0, int c0, f32x4 v, int lane) {
    typename MM::ET* q = dst + (c0 + (lane & 15)) * ld + r0 + 4 * (lane >> 4);
    if constexpr (sizeof(typename MM::ET) == 2) {
        u16x4 u;
#pragma unroll
        for (int r = 0; r < 4; ++r) u[r] = MM::from_f32(v[r]);
        *reinterpret_cast<u16x4*>(q) = u;
    } else {
        *reinterpret_cast<f32x4*>(q) = v;
    }
}
template <class MM>
__device__ __forceinline__ f32x4 gemm(const typename MM::ET* A, int lda, int m0, const typename MM::ET* Bt, int ldb,
                                      int n0, int k0, int k1, f32x4 acc, int lane) {
    for (int k = k0; k < k1; k += MM::KS)
        acc = MM::mma(MM::load(A, lda, m0, k, lane), MM::load(Bt, ldb, n0, k, lane), acc);
    return acc;
}

// N fp32 values rounded to the element type ET, in 16-byte vectors (the
// rounding of store_row), and the store of such vectors.
template <typename ET, int N>
__device__ __forceinline__ void pack_row(const float* src, f32x4* dst) {
    if constexpr (sizeof(ET) == 2) {
#pragma unroll
        for (int m = 0; m < N / 8; ++m) {
            u16x8 u;
#pragma unroll
            for (int e = 0; e < 8; ++e) u[e] = f32_to_bf16_bits(src[8 * m + e]);
            dst[m] = __builtin_bit_cast(f32x4, u);
        }
    } else {
#pragma unroll
        for (int m = 0; m < N / 4; ++m) dst[m] = f32x4{src[4 * m], src[4 * m + 1], src[4 * m + 2], src[4 * m + 3]};
    }
}
template <typename ET, int N>
__device__ __forceinline__ void store_packed(ET* dst, const f32x4* v) {
    constexpr int E = 16 / static_cast<int>(sizeof(ET));
#pragma unroll
    for (int m = 0; m < N / E; ++m) *reinterpret_cast<f32x4*>(dst + E * m) = v[m];
}

// Widen N elements held as loaded (16-byte vectors of IT) to fp32.
template <typename IT, int N>
__device__ __forceinline__ void widen_row(const f32x4* r, float* dst) {
    if constexpr (sizeof(IT) == 2) {
#pragma unroll
        for (int m = 0; m < N / 8; ++m) {
            const u16x8 u = __builtin_bit_cast(u16x8, r[m]);
#pragma unroll
            for (int e = 0; e < 8; ++e) dst[8 * m + e] = bf16_bits_to_f32(u[e]);
        }
    } else {
#pragma unroll
        for (int m = 0; m < N / 4; ++m)
#pragma unroll
            for (int e = 0; e < 4; ++e) dst[4 * m + e] = r[m][e];
    }
}

// MFMA operands for a product whose B operand is a row-major [k][n] LDS tile.
// bf16: B is read with the transposing LDS read (lane (n, g), g = lane / 16,
// receives rows k0 + 4g .. + 3 and k0 + 16 + 4g .. + 3 of column n0 + n), and
// the A fragment supplies the same contraction indices.  fp32: one element
// per lane, k = k0 + lane / 16.
template <class MM>
__device__ __forceinline__ typename MM::Frag load_ap(const typename MM::ET* base, int ld, int r0, int k0, int lane) {
    if constexpr (sizeof(typename MM::ET) == 2) {
        const uint16_t* row = base + (r0 + (lane & 15)) * ld + k0 + 4 * (lane >> 4);
        const u16x4 lo = *reinterpret_cast<const u16x4*>(row);
        const u16x4 hi = *reinterpret_cast<const u16x4*>(row + 16);
        const u16x8 u = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        return __builtin_bit_cast(typename MM::Frag, u);
    } else {
        return MM::load(base, ld, r0, k0, lane);
    }
}
template <class MM>
__device__ __forceinline__ typename MM::Frag load_kn(const typename MM::ET* base, int ld, int k0, int n0, int lane) {
    if constexpr (sizeof(typename MM::ET) == 2) {
        const int i = lane & 15, g = lane >> 4;
        const uint16_t* a0 = base + (k0 + 4 * g + (i >> 2)) * ld + n0 + 4 * (i & 3);
        const bf16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)a0);
        const bf16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(a0 + 16 * ld));
        return typename MM::Frag{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    } else {
        return base[(k0 + (lane >> 4)) * ld + n0 + (lane & 15)];
    }
}

// ------------------------------------------------------------------ prep
// Threads of a prep workgroup: its LDS allows one workgroup per CU, so wide
// channels take 8 waves (two per SIMD) to overlap the latency of one wave's
// LDS and memory chains with another's work.
__host__ __device__ constexpr int prep_threads(int K) { return K >= 64 ? 512 : 256; }

template <int K, bool BF, bool BWD, int V = K>
struct PrepSmem {
    using ET = typename Mma<BF>::ET;
    static constexpr int LDE = K + Mma<BF>::PAD;
    float G[kChunk][K + 4];  // 16-byte aligned rows
    union alignas(16) {
        struct {
            ET qL[kChunk][LDE];   // q^ exp(G_i - G_ref(I))
            ET kL[kChunk][LDE];   // k^ exp(G_i - G_ref(I))
            ET kbe[kChunk][LDE];  // k^ exp(G_end(J) - G_j)
        } op;
        float T[kChunk][kChunk + 4];  // 16-byte aligned rows (MFMA A operand)
        struct {
            ET TB[kChunk][kChunk + Mma<BF>::PAD];  // T diag(beta): A operand of W and U
            ET KE[kChunk][K + Mma<BF>::PAD];       // k^ exp(G), row-major (B operand, read transposed)
            ET Vr[kChunk][V + Mma<BF>::PAD];       // v, row-major (B operand, read transposed)
        } wu;
    } u;
    float A[kChunk][kChunk + 4];  // 16-byte aligned rows (MFMA A operand)
    float M[kChunk][kChunk + 1];
    ET Ak[BWD ? kChunk : 1][kChunk + 1];  // un-scaled k-k scores (backward only), as stored
    float P[4][K];     // exp(G_end(I) - G_ref(I)): decay across sub-block I
    float invP[4][K];  // 1 / P (finite where the block is factorised)
    float Er[4][K];    // exp(G_ref(I))
    float Ec[4][K];    // exp(G_last - G_end(I))
    float F20[K];      // P_1:      sub-block pair (2, 0)
    float F30[K];      // P_1 P_2:  pair (3, 0)
    float F31[K];      // P_2:      pair (3, 1)
    float gC[K];
    float rq[kChunk], rk[kChunk], beta[kChunk];
    float X[3][kSub][kSub + 1];
    int unsafe[4];
};

// Persistent grid of the prep kernel: as many workgroups as fit on the 256
// CUs at once (160 KiB of LDS and 2048 threads per CU), at most one per item.
template <int K, bool BF, bool BWD, int V = K>
__host__ inline unsigned prep_grid(int64_t n_items) {
    constexpr size_t lds = sizeof(PrepSmem<K, BF, BWD, V>);
    constexpr int by_lds = static_cast<int>((160 * 1024) / lds);
    constexpr int by_threads = 2048 / prep_threads(K);
    constexpr int per_cu = by_lds < by_threads ? by_lds : by_threads;
    const int64_t cap = static_cast<int64_t>(kPersistentGrid) * (per_cu > 0 ? per_cu : 1);
    return static_cast<unsigned>(n_items < cap ? n_items : cap);
}

// BWD additionally writes T = (I + A)^-1 and the un-scaled strictly lower
// k-k score matrix (BwdExtra layout) for the backward kernels.
//
// Persistent over the (slot, head) items, item = slot * H + h: workgroup b
// takes items b, b + gridDim.x, ...  While an item computes, the next item's
// q, k, g and beta (requested once the prologue has consumed the current
// ones) and v (requested once the current v is in LDS) are in flight, and
// the current item's stores drain behind the next item's work.
template <int K, bool BF, bool BWD, int V = K>
__global__ __launch_bounds__(prep_threads(K)) void chunk_prep_kernel(ChunkParams p, const int32_t* chunk_off,
                                                              uint8_t* ws, int64_t slot_bytes, int64_t n_items) {
    using MM = Mma<BF>;
    using ET = typename MM::ET;
    using IT = typename std::conditional<BF, uint16_t, float>::type;  // q/k/v element
    using L = PrepLayout<K, BF, V>;
    using X = BwdExtra<K, BF, V>;
    constexpr int NT = prep_threads(K);
    constexpr int NW = NT / 64;     // waves
    constexpr int TPR = NT / kChunk;  // threads per row in row-wise phases
    constexpr int CPT = K / TPR;      // channels per thread in row-wise phases
    static_assert(CPT % 8 == 0, "row segments are whole 16-byte vectors");
    constexpr int CPTV = V / TPR;     // value channels per thread
    static_assert(CPTV % 8 == 0, "row segments are whole 16-byte vectors");
    constexpr int LDE = PrepSmem<K, BF, BWD, V>::LDE;
    __shared__ __attribute__((aligned(16))) PrepSmem<K, BF, BWD, V> s;

    const int H = p.H;
    const int64_t GS = gridDim.x;
    constexpr int VEI = 16 / static_cast<int>(sizeof(IT));  // q/k/v elements per 16-byte vector
    constexpr int NQV = CPT / VEI;
    constexpr int NGV = CPT / 4;
    constexpr int NVV = CPTV / VEI;
    const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
    // slot-map entry of an item (packed input; unused for dense input)
    auto map_entry = [&](int64_t item) -> int4 {
        int4 e = {-1, 0, 0, 0};
        if (p.cu_seqlens && item < n_items)
            e = reinterpret_cast<const int4*>(reinterpret_cast<const uint8_t*>(chunk_off) + plan_map_offset(p.N))[item / H];
        return e;
    };
    auto decode = [&](int64_t item, int4 e, int& n, int& j, int64_t& start, int& len) -> bool {
        if (item >= n_items) return false;
        if (p.cu_seqlens) {
            n = e.x;
            j = e.y;
            start = e.z;
            len = e.w;
            return n >= 0;
        }
        const int nc = n_chunks(p.T);
        const int slot = static_cast<int>(item / H);
        n = slot / nc;
        j = slot % nc;
        start = static_cast<int64_t>(n) * p.T;
        len = p.T;
        return n < p.N;
    };
    // this thread's raw inputs of one item (row i, channel parts pq)
    f32x4 qraw[NQV], kraw[NQV], graw[NGV], vraw[NVV];
    float braw = 0.f;
    auto fetch_qkgb = [&](bool ok, int64_t rowh, int i_, int pq_, int rows_) {
        const bool vr = ok && i_ < rows_;
        const IT* qs = static_cast<const IT*>(p.q) + rowh * K + pq_ * CPT;
        const IT* ks = static_cast<const IT*>(p.k) + rowh * K + pq_ * CPT;
        const float* gs = p.g + rowh * K + pq_ * CPT;
#pragma unroll
        for (int m = 0; m < NQV; ++m) {
            qraw[m] = vr ? *reinterpret_cast<const f32x4*>(qs + VEI * m) : zero4;
            kraw[m] = vr ? *reinterpret_cast<const f32x4*>(ks + VEI * m) : zero4;
        }
#pragma unroll
        for (int m = 0; m < NGV; ++m) graw[m] = vr ? *reinterpret_cast<const f32x4*>(gs + 4 * m) : zero4;
        braw = vr ? p.beta[rowh] : 0.f;
    };
    auto fetch_v = [&](bool ok, int64_t rowh, int i_, int pq_, int rows_) {
        const bool vr = ok && i_ < rows_;
        const IT* vs = static_cast<const IT*>(p.v) + rowh * V + pq_ * CPTV;
#pragma unroll
        for (int m = 0; m < NVV; ++m) vraw[m] = vr ? *reinterpret_cast<const f32x4*>(vs + VEI * m) : zero4;
    };

    // the first item: its inputs, waited for here (so that the loop's waits
    // only ever count requests made one item earlier)
    int4 mcur = map_entry(blockIdx.x);
    int4 mnext = map_entry(blockIdx.x + GS);
    {
        int n0 = 0, j0 = 0, len0 = 0;
        int64_t st0 = 0;
        const bool ok0 = decode(blockIdx.x, mcur, n0, j0, st0, len0);
        const int i0 = static_cast<int>(threadIdx.x) / TPR, pq0 = static_cast<int>(threadIdx.x) % TPR;
        const int rows0 = ok0 ? min(kChunk, len0 - j0 * kChunk) : 0;
        const int64_t rowh0 = (st0 + static_cast<int64_t>(j0) * kChunk + i0) * H +
                              item_head(blockIdx.x, H, GS, p.gate_mode != GATE_LOGDECAY);
        fetch_qkgb(ok0, rowh0, i0, pq0, rows0);
        fetch_v(ok0, rowh0, i0, pq0, rows0);
#pragma unroll
        for (int m = 0; m < NQV; ++m) asm volatile("" ::"v"(qraw[m]), "v"(kraw[m]));
#pragma unroll
        for (int m = 0; m < NGV; ++m) asm volatile("" ::"v"(graw[m]));
#pragma unroll
        for (int m = 0; m < NVV; ++m) asm volatile("" ::"v"(vraw[m]));
        asm volatile("" ::"v"(braw));
    }

    for (int64_t item = blockIdx.x; item < n_items; item += GS) {
    int n, j;
    int64_t start;
    int len;
    if (!decode(item, mcur, n, j, start, len)) break;  // items past the last chunk are all empty
    const int slot = static_cast<int>(item / H);
    const int h = item_head(item, H, GS, p.gate_mode != GATE_LOGDECAY);
    const int rows = min(kChunk, len - j * kChunk);  // >= 1 by construction

    // thread coordinates from an opaque copy of the thread id, so that the
    // body's per-thread LDS addresses are not hoisted out of the item loop
    // (each would hold a register for the whole loop)
    int tid = static_cast<int>(threadIdx.x);
    asm volatile("" : "+v"(tid));
    const int t = tid;
    const int lane = t & 63;
    const int w = t >> 6;
    uint8_t* out = ws + (static_cast<int64_t>(slot) * H + h) * slot_bytes;
    ET* gQE = reinterpret_cast<ET*>(out + L::kQE);
    ET* gKD = reinterpret_cast<ET*>(out + L::kKD);
    ET* gTB = reinterpret_cast<ET*>(out + L::kTB);
    ET* gMS = reinterpret_cast<ET*>(out + L::kMS);
    float* gGC = reinterpret_cast<float*>(out + L::kGC);

    // ---- 1. prologue, row-wise: thread -> (row i, quarter pq of the channels)
    const int i = t / TPR;
    const int pq = t % TPR;
    const int c0 = pq * CPT;
    const int cv0 = pq * CPTV;
    const bool valid = i < rows;
    float qh[CPT], kh[CPT], gv[CPT];
    widen_row<IT, CPT>(qraw, qh);
    widen_row<IT, CPT>(kraw, kh);
    widen_row<float, CPT>(graw, gv);
    float ssq = 0.f, ssk = 0.f;
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
        ssq += qh[c] * qh[c];
        ssk += kh[c] * kh[c];
    }
#pragma unroll
    for (int o = 1; o < TPR; o <<= 1) {
        ssq += __shfl_xor(ssq, o, 64);
        ssk += __shfl_xor(ssk, o, 64);
    }
    float rq = 1.f, rk = 1.f;
    if (p.use_qk_l2norm) {
        rq = rsqrtf(ssq + kL2Eps);
        rk = rsqrtf(ssk + kL2Eps);
    }
    if (!valid) rq = rk = 0.f;
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
        qh[c] *= rq;
        kh[c] *= rk;
    }
    if (valid && p.gate_mode != GATE_LOGDECAY) {
        const float rate = __expf(p.A_log[h]);
        float bias[CPT];  // requested as whole vectors, waited for once
        if (p.dt_bias) {
            load_row<CPT>(p.dt_bias + h * K + c0, bias);
        } else {
#pragma unroll
            for (int c = 0; c < CPT; ++c) bias[c] = 0.f;
        }
#pragma unroll
        for (int c = 0; c < CPT; ++c) gv[c] = gate_eff(p.gate_mode, gv[c], rate, bias[c], p.lower_bound);
    }
    store_row<CPT>(&s.G[i][c0], gv);
    if (pq == 0) {
        s.rq[i] = rq;
        s.rk[i] = rk;
        float b = braw;
        if (valid && p.use_beta_sigmoid) b = sigmoidf_(b);
        s.beta[i] = b;
    }
    // the next item: where it is, and its q, k, g and beta (this item's are
    // consumed); the slot-map entry of the item after it
    int nn = 0, jn = 0, lenn = 0;
    int64_t stn = 0;
    const bool okn = decode(item + GS, mnext, nn, jn, stn, lenn);
    const int rowsn = okn ? min(kChunk, lenn - jn * kChunk) : 0;
    const int64_t rowhn = (stn + static_cast<int64_t>(jn) * kChunk + i) * H +
                          item_head(item + GS, H, GS, p.gate_mode != GATE_LOGDECAY);
    const int4 mnext2 = map_entry(item + 2 * GS);
    fetch_qkgb(okn, rowhn, i, pq, rowsn);
    asm volatile("" ::: "memory");  // keeps the requests here (not sunk to the loop's end)
    if (t < 4) s.unsafe[t] = 0;
    // A, M and Ak are not cleared: every entry that step 6 or 7 reads is
    // written in step 5 (blocks above the diagonal are masked in step 7)
    __syncthreads();

    // ---- 2. inclusive cumulative sum over the 64 rows, per channel
    {
        constexpr int SEGS = NT / K;      // row segments per channel
        constexpr int SEGLEN = kChunk / SEGS;
        const int c = t % K;
        const int sg = t / K;
        float acc = 0.f;
        for (int r = sg * SEGLEN; r < (sg + 1) * SEGLEN; ++r) {
            acc += s.G[r][c];
            s.G[r][c] = acc;
        }
        __syncthreads();
        float off = 0.f;
        for (int q = 0; q < sg; ++q) off += s.G[(q + 1) * SEGLEN - 1][c];
        __syncthreads();
        if (sg > 0)
            for (int r = sg * SEGLEN; r < (sg + 1) * SEGLEN; ++r) s.G[r][c] += off;
    }
    __syncthreads();

    // ---- 3. per-channel sub-block factors
    for (int c = t; c < K; c += NT) {
        float Gref[4], Gend[4];
#pragma unroll
        for (int I = 0; I < 4; ++I) {
            Gref[I] = I == 0 ? 0.f : s.G[kSub * I - 1][c];
            Gend[I] = s.G[kSub * I + kSub - 1][c];
        }
        const float Glast = Gend[3];
#pragma unroll
        for (int I = 0; I < 4; ++I) {
            const float span = Gref[I] - Gend[I];  // >= 0 for decays
            s.P[I][c] = __expf(-span);
            s.invP[I][c] = __expf(span);
            s.Er[I][c] = __expf(Gref[I]);
            s.Ec[I][c] = __expf(Glast - Gend[I]);
            if (!(span <= kSpanLimit)) s.unsafe[I] = 1;  // also catches NaN
        }
        s.F20[c] = s.P[1][c];
        s.F31[c] = s.P[2][c];
        s.F30[c] = s.P[1][c] * s.P[2][c];
        s.gC[c] = __expf(Glast);
    }
    __syncthreads();

    // ---- 4. factored operands (LDS) and the chunk's outputs QE, KD (and KE);
    //         those three are stored after step 5's products are issued, and
    //         k^ exp(G) stays in registers for W
    constexpr int PV = CPT * static_cast<int>(sizeof(ET)) / 16;
    f32x4 pQE[PV], pKE[PV], pKD[PV];
    {
        const int I = i / kSub;
        float a_[CPT], e_[CPT], o_[CPT];
#pragma unroll
        for (int c = 0; c < CPT; ++c) {
            const float Gi = s.G[i][c0 + c];
            const float Gr = I == 0 ? 0.f : s.G[kSub * I - 1][c0 + c];
            const float Ge = s.G[kSub * I + kSub - 1][c0 + c];
            a_[c] = __expf(Gi - Gr);
            e_[c] = __expf(Ge - Gi);
        }
#pragma unroll
        for (int c = 0; c < CPT; ++c) o_[c] = qh[c] * a_[c];
        store_row<CPT>(&s.u.op.qL[i][c0], o_);
#pragma unroll
        for (int c = 0; c < CPT; ++c) o_[c] = kh[c] * a_[c];
        store_row<CPT>(&s.u.op.kL[i][c0], o_);
#pragma unroll
        for (int c = 0; c < CPT; ++c) o_[c] = kh[c] * e_[c];
        store_row<CPT>(&s.u.op.kbe[i][c0], o_);
#pragma unroll
        for (int c = 0; c < CPT; ++c) o_[c] = p.scale * qh[c] * a_[c] * s.Er[I][c0 + c];
        pack_row<ET, CPT>(o_, pQE);
#pragma unroll
        for (int c = 0; c < CPT; ++c) o_[c] = kh[c] * a_[c] * s.Er[I][c0 + c];
        pack_row<ET, CPT>(o_, pKE);
#pragma unroll
        for (int c = 0; c < CPT; ++c) o_[c] = kh[c] * e_[c] * s.Ec[I][c0 + c];
        pack_row<ET, CPT>(o_, pKD);
    }
    __syncthreads();

    // Level job of diagonal sub-block I (one wave): the pairs of level hh of the
    // level decomposition (level_pair; hh = 0: the diagonal) of A (and the
    // un-scaled Ak) and M, from the normalised q and k rows that step 5 leaves
    // in the qL and kL tiles, each element times its factor (at most 1).
    auto level_job = [&](int hh, int I, int lane_) {
        const int pr = lane_ & 15;  // this lane's operand row in the block
        const int row = kSub * I + pr;
        const bool later = hh == 0 || (pr & hh), earlier = hh == 0 || !(pr & hh);
        const int ref = hh == 0 ? row : kSub * I + (pr & ~(2 * hh - 1)) + hh - 1;
        f32x4 accM = {0.f, 0.f, 0.f, 0.f}, accA = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 2
        for (int k0 = 0; k0 < K; k0 += MM::KS) {
            const int ch = k0 + (lane_ >> 4) * MM::KPL;
            float fa[MM::KPL], fb[MM::KPL];
#pragma unroll
            for (int e = 0; e < MM::KPL; ++e) {
                const float f = hh == 0 ? 1.f : level_fac(pr, hh, s.G[row][ch + e], s.G[ref][ch + e]);
                fa[e] = later ? f : 0.f;
                fb[e] = earlier ? f : 0.f;
            }
            const auto xq = MM::load(&s.u.op.qL[0][0], LDE, kSub * I, k0, lane_);
            const auto xk = MM::load(&s.u.op.kL[0][0], LDE, kSub * I, k0, lane_);
            const auto bK = MM::scale(xk, fb);
            accM = MM::mma(MM::scale(xq, fa), bK, accM);
            if (hh) accA = MM::mma(MM::scale(xk, fa), bK, accA);
        }
        const int b_ = lane_ & 15, colg = kSub * I + b_;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int a_ = 4 * (lane_ >> 4) + r, rowg = kSub * I + a_;
            if (hh == 0 ? a_ == b_ : level_pair(a_, b_, hh)) {
                s.M[rowg][colg] = accM[r];
                s.A[rowg][colg] = accA[r] * s.beta[rowg];  // 0 on the diagonal
                if (BWD) s.Ak[rowg][colg] = MM::from_f32(accA[r]);
            }
        }
    };

    // ---- 5. A and M sub-block tiles on MFMA (job = (matrix, I, J<=I)); 20 jobs,
    //         then for each diagonal sub-block too wide to factorise through one
    //         reference row, its level jobs (level_job: levels 8, 4, 2, 1 and the
    //         diagonal)
    for (int job = w; job < 20; job += NW) {
        const bool isM = job >= 10;
        int tj = isM ? job - 10 : job;
        int I = 0;
        while (tj > I) { tj -= I + 1; ++I; }
        const int J = tj;
        if (J == I && s.unsafe[I]) continue;  // formed by its level jobs
        const float* fac = nullptr;
        if (J == I) fac = s.invP[I];
        else if (I == 2 && J == 0) fac = s.F20;
        else if (I == 3 && J == 0) fac = s.F30;
        else if (I == 3 && J == 1) fac = s.F31;
        const ET* Lop = isM ? &s.u.op.qL[0][0] : &s.u.op.kL[0][0];
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
        for (int k0 = 0; k0 < K; k0 += MM::KS) {
            auto a = MM::load(Lop, LDE, kSub * I, k0, lane);
            auto b = MM::load(&s.u.op.kbe[0][0], LDE, kSub * J, k0, lane);
            if (fac) b = MM::scale(b, fac + k0 + (lane >> 4) * MM::KPL);
            acc = MM::mma(a, b, acc);
        }
        const int col = kSub * J + (lane & 15);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = kSub * I + 4 * (lane >> 4) + r;
            float v = acc[r];
            if (isM) {
                if (J == I && col > row) v = 0.f;
                s.M[row][col] = v;
            } else {
                if (J == I && col >= row) v = 0.f;
                s.A[row][col] = v * s.beta[row];
                if (BWD) s.Ak[row][col] = MM::from_f32(v);
            }
        }
    }
    store_packed<ET, CPT>(gQE + i * K + c0, pQE);
    if (BWD) store_packed<ET, CPT>(reinterpret_cast<ET*>(out + X::kKE) + i * K + c0, pKE);
    store_packed<ET, CPT>(gKD + i * K + c0, pKD);
    if (s.unsafe[0] | s.unsafe[1] | s.unsafe[2] | s.unsafe[3]) {  // uniform
        __syncthreads();  // the factored tiles are read
        store_row<CPT>(&s.u.op.qL[i][c0], qh);
        store_row<CPT>(&s.u.op.kL[i][c0], kh);
        __syncthreads();
        for (int job = w; job < 20; job += NW) {
            const int I = job / 5, lv = job % 5;
            if (s.unsafe[I]) level_job(lv < 4 ? (8 >> lv) : 0, I, lane);
        }
    }
    __syncthreads();

    // ---- 6. T = (I + A)^-1: diagonal sub-blocks by forward substitution ...
    // (T above the diagonal is never read before step 7, which masks it).
    // Lane jc solves column jc: x_r = [r == jc] - sum_{m < r} A_rm x_m.  The
    // sums are formed column by column (each x_m, once known, enters every
    // later row's sum at once), so the dependent chain is one product per
    // row rather than the whole sum; every sum still adds its terms in the
    // order m = 0, 1, ...
    if (w < 4 && lane < kSub) {
        const int I = w;
        const int jc = lane;
        float x[kSub], acc[kSub];
#pragma unroll
        for (int r = 0; r < kSub; ++r) acc[r] = 0.f;
#pragma unroll
        for (int m = 0; m < kSub; ++m) {
            x[m] = m < jc ? 0.f : (m == jc ? 1.f : -acc[m]);
#pragma unroll
            for (int r = m + 1; r < kSub; ++r) acc[r] += s.A[kSub * I + r][kSub * I + m] * x[m];
        }
#pragma unroll
        for (int r = 0; r < kSub; ++r) s.u.T[kSub * I + r][kSub * I + jc] = x[r];
    }
    __syncthreads();
    // ... then the off-diagonal sub-blocks by distance d = I - J: T_IJ = -T_II
    // sum_L A_IL T_LJ.  Wave w forms block (d + w, w) as two fp32 16 x 16 x 16
    // MFMA products: lane (lc, lg) supplies A[lc][4 lg + st] and B[4 lg + st][lc]
    // at step st, and holds rows 4 lg + r of column lc of the result.
    for (int d = 1; d < 4; ++d) {
        if (w < 4 - d) {
            const int J = w, I = d + w, lc = lane & 15, lg = lane >> 4;
            f32x4 x = {0.f, 0.f, 0.f, 0.f};
            for (int Lb = J; Lb < I; ++Lb) {
                const float4 a4 = *reinterpret_cast<const float4*>(&s.A[kSub * I + lc][kSub * Lb + 4 * lg]);
                const float* tc = &s.u.T[kSub * Lb + 4 * lg][kSub * J + lc];
                x = __builtin_amdgcn_mfma_f32_16x16x4f32(a4.x, tc[0 * (kChunk + 4)], x, 0, 0, 0);
                x = __builtin_amdgcn_mfma_f32_16x16x4f32(a4.y, tc[1 * (kChunk + 4)], x, 0, 0, 0);
                x = __builtin_amdgcn_mfma_f32_16x16x4f32(a4.z, tc[2 * (kChunk + 4)], x, 0, 0, 0);
                x = __builtin_amdgcn_mfma_f32_16x16x4f32(a4.w, tc[3 * (kChunk + 4)], x, 0, 0, 0);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) s.X[w][4 * lg + r][lc] = x[r];  // read back by this wave only
            const float4 t4 = *reinterpret_cast<const float4*>(&s.u.T[kSub * I + lc][kSub * I + 4 * lg]);
            f32x4 y = {0.f, 0.f, 0.f, 0.f};
            y = __builtin_amdgcn_mfma_f32_16x16x4f32(t4.x, s.X[w][4 * lg + 0][lc], y, 0, 0, 0);
            y = __builtin_amdgcn_mfma_f32_16x16x4f32(t4.y, s.X[w][4 * lg + 1][lc], y, 0, 0, 0);
            y = __builtin_amdgcn_mfma_f32_16x16x4f32(t4.z, s.X[w][4 * lg + 2][lc], y, 0, 0, 0);
            y = __builtin_amdgcn_mfma_f32_16x16x4f32(t4.w, s.X[w][4 * lg + 3][lc], y, 0, 0, 0);
#pragma unroll
            for (int r = 0; r < 4; ++r) s.u.T[kSub * I + 4 * lg + r][kSub * J + lc] = -y[r];
        }
        __syncthreads();
    }

    // ---- 7. T diag(beta) and scale * M to the workspace; thread t owns EPT
    //         consecutive entries of one row (entries above the diagonal are
    //         zero: they were never written in LDS)
    constexpr int EPT = kChunk * kChunk / NT;
    static_assert(EPT % 8 == 0, "whole 16-byte vectors per thread");
    const int e7 = t * EPT, a7 = e7 / kChunk, b7 = e7 % kChunk;
    float tbr[EPT];
    {
        float ms[EPT];
#pragma unroll
        for (int x = 0; x < EPT; ++x) {
            const int b = b7 + x;
            const bool up = b > a7;
            tbr[x] = up ? 0.f : s.u.T[a7][b] * s.beta[b];
            ms[x] = up ? 0.f : p.scale * s.M[a7][b];
        }
        store_row<EPT>(gTB + e7, tbr);
        store_row<EPT>(gMS + e7, ms);
    }
    for (int c = t; c < K; c += NT) gGC[c] = s.gC[c];
    if (BWD) {
        float tt[EPT], ak[EPT];
#pragma unroll
        for (int x = 0; x < EPT; ++x) {
            const int b = b7 + x;
            tt[x] = b > a7 ? 0.f : s.u.T[a7][b];
            ak[x] = b >= a7 ? 0.f : MM::to_f32(s.Ak[a7][b]);
        }
        store_row<EPT>(reinterpret_cast<ET*>(out + X::kT) + e7, tt);
        store_row<EPT>(reinterpret_cast<ET*>(out + X::kAK) + e7, ak);
    }
    __syncthreads();

    // ---- 8. the WY pair W = T diag(beta) (k^ exp(G)), U = T diag(beta) v on MFMA
    {
        constexpr int LDC = kChunk + MM::PAD;
        store_row<EPT>(&s.u.wu.TB[a7][b7], tbr);
        // KE and v rows as they are (v exactly as loaded: IT is ET)
        store_packed<ET, CPT>(&s.u.wu.KE[i][c0], pKE);
#pragma unroll
        for (int m = 0; m < NVV; ++m) *reinterpret_cast<f32x4*>(&s.u.wu.Vr[i][cv0 + VEI * m]) = vraw[m];
        fetch_v(okn, rowhn, i, pq, rowsn);
        asm volatile("" ::: "memory");
        __syncthreads();
        ET* gW = reinterpret_cast<ET*>(out + L::kW);
        ET* gU = reinterpret_cast<ET*>(out + L::kU);
        // wave w: row tile w % 4, every (NW / 4)-th column tile from w / 4;
        // W has K / 16 column tiles and U has V / 16
        constexpr int NCTWU = (K > V ? K : V) / 16;
        const int rt = w & 3;
#pragma unroll 2
        for (int ct = w >> 2; ct < NCTWU; ct += NW / 4) {
            f32x4 aw = {0.f, 0.f, 0.f, 0.f}, au = {0.f, 0.f, 0.f, 0.f};
            for (int k0 = 0; k0 < 16 * (rt + 1); k0 += MM::KS) {
                const auto a = load_ap<MM>(&s.u.wu.TB[0][0], LDC, 16 * rt, k0, lane);
                if (K == V || ct < K / 16) aw = MM::mma(a, load_kn<MM>(&s.u.wu.KE[0][0], LDE, k0, 16 * ct, lane), aw);
                if (K == V || ct < V / 16) au = MM::mma(a, load_kn<MM>(&s.u.wu.Vr[0][0], V + MM::PAD, k0, 16 * ct, lane), au);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 16 * rt + 4 * (lane >> 4) + r, col = 16 * ct + (lane & 15);
                if (K == V || ct < K / 16) gW[row * K + col] = MM::from_f32(aw[r]);
                if (K == V || ct < V / 16) gU[row * V + col] = MM::from_f32(au[r]);
            }
        }
    }
    mcur = mnext;
    mnext = mnext2;
    }  // items
}

// ------------------------------------------------------------------ state
// Copy a [R][C] global matrix into LDS rows of leading dimension ld, with NT
// threads; every load is issued before the first store.
template <typename ET, int R, int C, int NT = kThreads>
__device__ __forceinline__ void copy_in(ET* dst, int ld, const ET* src, int t) {
    constexpr int VE = 16 / sizeof(ET);  // elements per 16-byte vector
    constexpr int NV = R * C / VE;
#pragma unroll
    for (int m = 0; m < (NV + NT - 1) / NT; ++m) {
        const int e = t + m * NT;
        if (NV % NT != 0 && e >= NV) break;
        const int r = (e * VE) / C, c = (e * VE) % C;
        const f32x4 v = *reinterpret_cast<const f32x4*>(src + r * C + c);
        *reinterpret_cast<f32x4*>(dst + r * ld + c) = v;
    }
}
// Same, transposed: dst[c][r] = src[r][c].  Consecutive threads take
// consecutive rows, so the scattered LDS stores of a wavefront land on
// consecutive addresses.
template <typename ET, int R, int C, int NT = kThreads>
__device__ __forceinline__ void copy_in_t(ET* dst, int ld, const ET* src, int t) {
    constexpr int VE = 16 / sizeof(ET);
    constexpr int NV = R * C / VE;
#pragma unroll
    for (int m = 0; m < (NV + NT - 1) / NT; ++m) {
        const int e = t + m * NT;
        if (NV % NT != 0 && e >= NV) break;
        const int r = e % R, c = (e / R) * VE;
        const f32x4 v = *reinterpret_cast<const f32x4*>(src + r * C + c);
        const ET* ve = reinterpret_cast<const ET*>(&v);
#pragma unroll
        for (int x = 0; x < VE; ++x) dst[(c + x) * ld + r] = ve[x];
    }
}

// A [R][C] block (row stride `stride` elements in global memory) moved
// global -> registers -> LDS in 16-byte vectors, so that the load of the next
// chunk's block can be issued before the current chunk's work and consumed
// after it.  TRANS stores the block transposed (dst[c][r]); rows at or past
// `rows` load as zero.
template <typename ET, int R, int C, bool TRANS, int NT = kThreads>
struct Seg {
    static constexpr int VE = 16 / sizeof(ET);
    static constexpr int NV = R * C / VE;
    static constexpr int PER = (NV + NT - 1) / NT;
    f32x4 r[PER];
    __device__ __forceinline__ static void at(int e, int& row, int& col) {
        if (TRANS) {
            row = e % R;
            col = (e / R) * VE;
        } else {
            row = (e * VE) / C;
            col = (e * VE) % C;
        }
    }
    __device__ __forceinline__ void load(const ET* src, int64_t stride, int t, int rows = R) {
#pragma unroll
        for (int m = 0; m < PER; ++m) {
            const int e = t + m * NT;
            if (NV % NT == 0 || e < NV) {
                int row, col;
                at(e, row, col);
                if (row < rows) r[m] = *reinterpret_cast<const f32x4*>(src + row * stride + col);
                else r[m] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
        }
    }
    __device__ __forceinline__ void store(ET* dst, int ld, int t) const {
#pragma unroll
        for (int m = 0; m < PER; ++m) {
            const int e = t + m * NT;
            if (NV % NT == 0 || e < NV) {
                int row, col;
                at(e, row, col);
                if (TRANS) {
                    const ET* ve = reinterpret_cast<const ET*>(&r[m]);
#pragma unroll
                    for (int x = 0; x < VE; ++x) dst[(col + x) * ld + row] = ve[x];
                } else {
                    *reinterpret_cast<f32x4*>(dst + row * ld + col) = r[m];
                }
            }
        }
    }
};


// Forward state pass.  Per chunk, with the chunk's operands from its slot and
// the fp32 state S (K x BV columns of this workgroup) in MFMA accumulators:
//   WS = W S, D = U - WS, O = QE S + MS D, S = GC * S + KD^T D.
// STORE writes each chunk's entry state (BwdExtra::kS, transposed, element type ET) for
// the backward; WRITE_O computes and stores the output.  The next chunk's
// operands are prefetched into registers while the current chunk computes.
//
// GATE (with BV = V and 4 waves, so that a wave holds whole output rows)
// applies the full-rank output gate of the "atlas_core/kimi_k3/kda.rs" page
// (full_rank_output_gate) to each output row before it is stored: y =
// sigmoid(g) o / sqrt(mean_v(o^2) + eps), g the gate input p.out_gate.
template <int K, int V, int BV, bool BF, bool STORE, bool WRITE_O, int NT = kThreads, bool GATE = false>
__global__ __launch_bounds__(NT) void chunk_state_fwd_kernel(ChunkParams p, const int32_t* chunk_off,
                                                             uint8_t* ws, int64_t slot_bytes) {
    using MM = Mma<BF>;
    using ET = typename MM::ET;
    using IT = typename std::conditional<BF, uint16_t, float>::type;
    using L = PrepLayout<K, BF, V>;
    constexpr int LDK = K + MM::PAD;
    constexpr int LDC = kChunk + MM::PAD;
    constexpr int LDB = BV + MM::PAD;
    constexpr int NCT = BV / 16;
    constexpr int NST = (K / 16) * NCT;
    constexpr int NW = NT / 64;
    constexpr int SPW = (NST + NW - 1) / NW;
    constexpr int CSTEP = NW / 4;                 // waves per 16-row tile of the chunk
    constexpr int TW = (NCT + CSTEP - 1) / CSTEP;  // column tiles per wave
    constexpr int NVB = V / BV;
    constexpr int QR = WRITE_O ? kChunk : 0;  // rows of QE ahead of W in QW
    static_assert(!GATE || (BV == V && NT == kThreads && WRITE_O && !STORE),
                  "the gated output needs whole rows per wave");

    __shared__ __attribute__((aligned(16))) ET QW[QR + kChunk][LDK];   // [QE;] W
    __shared__ __attribute__((aligned(16))) ET KDt[K][LDC];
    __shared__ __attribute__((aligned(16))) ET MS[WRITE_O ? kChunk : 1][LDC];
    __shared__ __attribute__((aligned(16))) ET St[BV][LDK];
    __shared__ __attribute__((aligned(16))) ET Un[kChunk][LDB];
    __shared__ __attribute__((aligned(16))) ET Dt[BV][LDC];
    __shared__ __attribute__((aligned(16))) float gC[K];

    int chain, vb;
    if (!chain_of_block(blockIdx.x, p.N * p.H, NVB, chain, vb)) return;
    const int H = p.H;
    const int n = chain / H, h = chain % H;
    int64_t start;
    int len;
    seq_bounds(p, n, start, len);
    const int nc = chain_chunks(p, chunk_off, n, len);
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    // 16-row tile and first column tile of this wave (4 waves: every column tile)
    const int rw = NW > 4 ? (w & 3) : w, cw = NW > 4 ? (w >> 2) : 0;
    const int v0 = vb * BV;
    const int64_t slot0 = chunk_slot(p, chunk_off, n, 0);

    Seg<ET, kChunk, K, false, NT> sQE, sW;
    Seg<ET, kChunk, K, true, NT> sKD;
    Seg<ET, kChunk, kChunk, false, NT> sMS;
    Seg<ET, kChunk, BV, false, NT> sU;
    Seg<float, 1, K, false, NT> sGC;
    auto prefetch = [&](int jc) {
        const uint8_t* base = ws + ((slot0 + jc) * H + h) * slot_bytes;
        if (WRITE_O) sQE.load(reinterpret_cast<const ET*>(base + L::kQE), K, t);
        sW.load(reinterpret_cast<const ET*>(base + L::kW), K, t);
        sKD.load(reinterpret_cast<const ET*>(base + L::kKD), K, t);
        if (WRITE_O) sMS.load(reinterpret_cast<const ET*>(base + L::kMS), kChunk, t);
        sU.load(reinterpret_cast<const ET*>(base + L::kU) + v0, V, t);
        sGC.load(reinterpret_cast<const float*>(base + L::kGC), K, t);
    };

    // fp32 state tiles owned by this wave: tile m -> (row tile, col tile)
    f32x4 S[SPW];
    const int64_t sbase = (static_cast<int64_t>(n) * H + h) * K * V;
#pragma unroll
    for (int m = 0; m < SPW; ++m) {
        const int tt = w + NW * m;
        const int rt = tt / NCT, ct = tt % NCT;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            float v = 0.f;
            if (tt < NST && p.h0) v = p.h0[sbase + (16 * rt + 4 * (lane >> 4) + r) * V + v0 + 16 * ct + (lane & 15)];
            S[m][r] = v;
        }
    }

    IT* og = static_cast<IT*>(p.o);
    if (nc > 0) prefetch(0);
    for (int jc = 0; jc < nc; ++jc) {
        if (WRITE_O) sQE.store(&QW[0][0], LDK, t);
        sW.store(&QW[QR][0], LDK, t);
        sKD.store(&KDt[0][0], LDC, t);
        if (WRITE_O) sMS.store(&MS[0][0], LDC, t);
        sU.store(&Un[0][0], LDB, t);
        sGC.store(&gC[0], K, t);
        if (STORE) {
            uint8_t* base = ws + ((slot0 + jc) * H + h) * slot_bytes;
            ET* gS = reinterpret_cast<ET*>(base + BwdExtra<K, BF, V>::kS);
#pragma unroll
            for (int m = 0; m < SPW; ++m) {
                const int tt = w + NW * m;
                if (tt < NST) {
                    const int rt = tt / NCT, ct = tt % NCT;
                    tile_store_t<MM>(gS + v0 * K, K, 16 * rt, 16 * ct, S[m], lane);  // S^T rows
                }
            }
        }
#pragma unroll
        for (int m = 0; m < SPW; ++m) {
            const int tt = w + NW * m;
            if (tt < NST) tile_store_t<MM>(&St[0][0], LDK, 16 * (tt / NCT), 16 * (tt % NCT), S[m], lane);
        }
        __syncthreads();
        if (jc + 1 < nc) prefetch(jc + 1);

        // WS and (scale q exp(G)) S for this wave's 16 rows and column tiles
        f32x4 oq[TW], ws_[TW];
#pragma unroll
        for (int m = 0; m < TW; ++m) oq[m] = ws_[m] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 2
        for (int k0 = 0; k0 < K; k0 += MM::KS) {
            const auto aw = MM::load(&QW[0][0], LDK, QR + 16 * rw, k0, lane);
            typename MM::Frag aq{};
            if (WRITE_O) aq = MM::load(&QW[0][0], LDK, 16 * rw, k0, lane);
#pragma unroll
            for (int m = 0; m < TW; ++m) {
                const int ct = cw + CSTEP * m;
                if (ct < NCT) {
                    const auto b = MM::load(&St[0][0], LDK, 16 * ct, k0, lane);
                    ws_[m] = MM::mma(aw, b, ws_[m]);
                    if (WRITE_O) oq[m] = MM::mma(aq, b, oq[m]);
                }
            }
        }
        // D = U - W S
#pragma unroll
        for (int m = 0; m < TW; ++m) {
            const int ct = cw + CSTEP * m;
            if (ct < NCT) {
                f32x4 d;
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    d[r] = MM::to_f32(Un[16 * rw + 4 * (lane >> 4) + r][16 * ct + (lane & 15)]) - ws_[m][r];
                tile_store_t<MM>(&Dt[0][0], LDC, 16 * rw, 16 * ct, d, lane);
            }
        }
        __syncthreads();

        // O = scale (q exp(G)) S + scale M D
        if (WRITE_O) {
            for (int k0 = 0; k0 < 16 * (rw + 1); k0 += MM::KS) {
                const auto a = MM::load(&MS[0][0], LDC, 16 * rw, k0, lane);
#pragma unroll
                for (int m = 0; m < TW; ++m) {
                    const int ct = cw + CSTEP * m;
                    if (ct < NCT) oq[m] = MM::mma(a, MM::load(&Dt[0][0], LDC, 16 * ct, k0, lane), oq[m]);
                }
            }
            const int rbase = jc * kChunk;
            float rinv[4] = {1.f, 1.f, 1.f, 1.f};
            if constexpr (GATE) {  // each wave holds its 16 rows' whole V values
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float ss = 0.f;
#pragma unroll
                    for (int m = 0; m < TW; ++m) ss += oq[m][r] * oq[m][r];
                    rinv[r] = rsqrtf(row16_sum(ss) * (1.0f / V) + p.out_gate_eps);
                }
            }
#pragma unroll
            for (int m = 0; m < TW; ++m) {
                const int ct = cw + CSTEP * m;
                if (ct < NCT)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int row = 16 * rw + 4 * (lane >> 4) + r;
                        if (rbase + row < len) {
                            const int64_t oi = ((start + rbase + row) * H + h) * V + v0 + 16 * ct + (lane & 15);
                            float y = oq[m][r];
                            if constexpr (GATE) {
                                const float gi = p.out_gate_bf16 ? bf16_bits_to_f32(static_cast<const uint16_t*>(p.out_gate)[oi])
                                                                 : static_cast<const float*>(p.out_gate)[oi];
                                y = sigmoidf_(gi) * y * rinv[r];
                            }
                            Elem<IT>::store(og, oi, y);
                        }
                    }
            }
        }

        // S' = diag(exp(G_last)) S + (k exp(G_last - G))^T D
#pragma unroll
        for (int m = 0; m < SPW; ++m) {
            const int tt = w + NW * m;
            if (tt < NST) {
                const int rt = tt / NCT, ct = tt % NCT;
#pragma unroll
                for (int r = 0; r < 4; ++r) S[m][r] *= gC[16 * rt + 4 * (lane >> 4) + r];
#pragma unroll
                for (int k0 = 0; k0 < kChunk; k0 += MM::KS)
                    S[m] = MM::mma(MM::load(&KDt[0][0], LDC, 16 * rt, k0, lane),
                                   MM::load(&Dt[0][0], LDC, 16 * ct, k0, lane), S[m]);
            }
        }
        __syncthreads();
    }

    if (p.ht) {
#pragma unroll
        for (int m = 0; m < SPW; ++m) {
            const int tt = w + NW * m;
            if (tt < NST) {
                const int rt = tt / NCT, ct = tt % NCT;
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    p.ht[sbase + (16 * rt + 4 * (lane >> 4) + r) * V + v0 + 16 * ct + (lane & 15)] = S[m][r];
            }
        }
    }
}

// ------------------------------------------------------------------ state (producer/consumer)
// Forward state pass for K = V = 128 in bf16, BV value columns per workgroup
// (32 or 64), 64 (BV / 16 + 2) threads.  Waves 0 .. BV/16 - 1 (consumers) each
// own a 16-column strip of the fp32 state over all 128 rows, in MFMA
// accumulators.  Every product of a chunk
// step takes its B operand from registers: S itself, or D = U - W S formed
// in registers.  Its A operand is one of the chunk's operand tiles in LDS, read
// row-wise or transposed.  A consumer thus needs no other wave within a step.
// The last two waves (producers) do the global memory traffic: the next
// chunk's operand tiles go straight into the other half of a double-buffered
// LDS area, and the previous chunk's output rows (and, at BV = 32, its entry
// state) go out from LDS staging.  At BV = 64 the staged state would not fit
// the LDS beside the operand buffers, so each consumer stores its strip of the
// entry state itself, as 16-byte pieces of the transposed rows.  BV = 64 halves
// the workgroups per chain: when chains x 4 exceed the CUs, 32-column blocks
// would run in several rounds of workgroups, each as long as the chain.
// There is one barrier per chunk.
// Chunks ahead of use that the state passes warm L2 for.
constexpr int kWarmAhead = 4;
// With 64-column blocks twice as many chains share each XCD's L2, and four
// chunks ahead no longer fit it (B8 x T4096 forward state: 213 us at two
// chunks ahead, 228 at one, 231 at three, 237 at four).
constexpr int kWarmAhead64 = 2;

template <int BV>
struct StatePcFwd {
    static constexpr int oW = 0, oQE = 16384, oKD = 32768, oMS = 49152, oU = 57344, oGC = oU + 128 * BV;
    static constexpr int kBuf = oGC + 512;  // one chunk's operand tiles
};

// Threads of the producer/consumer state passes with BV value columns per workgroup.
__host__ __device__ constexpr int state_pc_threads(int BV) { return 64 * (BV / 16 + 2); }
// Value columns per workgroup of the producer/consumer state passes for
// `chains` (sequence, head) chains: 32 while four blocks per chain fit the
// CUs at one workgroup each (shorter chunk steps), else 64 (half as many
// rounds of workgroups, each as long as the whole chain).
__host__ __device__ constexpr int state_pc_bv(int chains) { return chains * 4 <= kPersistentGrid ? 32 : 64; }

template <bool STORE, bool WRITE_O, int BV = 32>
__global__ __launch_bounds__(state_pc_threads(BV)) void chunk_state_fwd_pc_kernel(ChunkParams p,
                                                                                  const int32_t* chunk_off,
                                                                                  uint8_t* ws, int64_t slot_bytes) {
    static_assert(BV == 32 || BV == 64, "32- or 64-column blocks");
    using Z = StatePcFwd<BV>;
    using L = PrepLayout<128, true>;
    constexpr int K = 128, V = 128, NVB = V / BV, NCW = BV / 16;
    constexpr bool STAGE_S = STORE && BV == 32;  // entry state staged for the producers
    constexpr int WA = BV == 32 ? kWarmAhead : kWarmAhead64;
    // L2 warm-up kWarmAhead chunks ahead (HBM latency exceeds a chunk step),
    // 128-byte lines split over the chain's
    // NVB workgroups, NWARM loads per producer lane
    constexpr int NL_OP = WRITE_O ? 384 : 256;                       // [QE,] W, KD
    constexpr int NL = NL_OP + (WRITE_O ? 64 : 0) + 128 + 4;         // + MS, U, GC
    constexpr int NWARM = (NL + NVB * 128 - 1) / (NVB * 128);
    // separate arrays, so that the compiler knows the staging and operand
    // reads do not alias the warm-up copies
    __shared__ __attribute__((aligned(1024))) uint8_t smb[2 * Z::kBuf];
    __shared__ __attribute__((aligned(1024))) uint8_t sms[STAGE_S ? 2 * 8192 : 16];  // S^T staging [32][128] per parity
    __shared__ __attribute__((aligned(1024))) uint8_t smo[2 * 128 * BV];  // O^T staging [BV][64] per parity
    __shared__ __attribute__((aligned(256))) uint8_t smj[256];

    int chain, vb;
    if (!chain_of_block(blockIdx.x, p.N * p.H, NVB, chain, vb)) return;
    const int H = p.H;
    const int n = chain / H, h = chain % H;
    int64_t start;
    int len;
    seq_bounds(p, n, start, len);
    const int nc = chain_chunks(p, chunk_off, n, len);
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int lg = lane >> 4, m = lane & 15;
    const int v0 = vb * BV;
    const int64_t slot0 = chunk_slot(p, chunk_off, n, 0);
    const int64_t sbase = (static_cast<int64_t>(n) * H + h) * K * V;
    const bool prod = w >= NCW;
    const int pw = w - NCW;
    auto slot = [&](int jc) { return ws + ((slot0 + jc) * H + h) * slot_bytes; };

    // ---- producer: chunk jc's operand tiles into buffer jc & 1 (57 + BV / 8 pieces of 1 KB)
    auto fetch = [&](int jc) {
        const uint8_t* base = slot(jc);
        uint8_t* buf = smb + (jc & 1) * Z::kBuf;
#pragma unroll
        for (int qq = 0; qq < 8; ++qq) {
            const int q = 2 * qq + pw;
            dma_tile_piece<128>(reinterpret_cast<const uint16_t*>(base + L::kW), K, buf + Z::oW, q, lane);
            dma_tile_piece<128>(reinterpret_cast<const uint16_t*>(base + L::kKD), K, buf + Z::oKD, q, lane);
            if (WRITE_O)
                dma_tile_piece<128>(reinterpret_cast<const uint16_t*>(base + L::kQE), K, buf + Z::oQE, q, lane);
        }
        if (WRITE_O)
#pragma unroll
            for (int qq = 0; qq < 4; ++qq)
                dma_tile_piece<64>(reinterpret_cast<const uint16_t*>(base + L::kMS), kChunk, buf + Z::oMS, 2 * qq + pw,
                                    lane);
#pragma unroll
        for (int qq = 0; qq < BV / 16; ++qq)
            dma_tile_piece<BV>(reinterpret_cast<const uint16_t*>(base + L::kU) + v0, V, buf + Z::oU, 2 * qq + pw, lane);
        if (pw == 1 && lane < 32) dma16(base + L::kGC + 16 * lane, buf + Z::oGC);
    };
    // ---- producer: chunk jc's entry state and output rows from staging jc & 1
    uint16_t* og = static_cast<uint16_t*>(p.o);
    auto drain = [&](int jc) {
        // every staging read first, then the stores.  The state goes out as
        // whole transposed rows (column v of S: 128 values, 256 bytes); the
        // output as 64-byte row segments, its staging read transposed twice
        // per lane for 8 columns.
        constexpr int NH = BV / 32;  // 32-column halves of the block
        const uint8_t* sts = sms + (jc & 1) * 8192;
        const uint8_t* sto = smo + (jc & 1) * (128 * BV);
        bf16x8 xs[4], xo[2][NH];
        if (STAGE_S)
#pragma unroll
            for (int q = 0; q < 4; ++q)  // S^T rows 16 pw + 4 q + lane / 16, 16-byte chunk lane % 16
                xs[q] = *reinterpret_cast<const bf16x8*>(sts + swz_off<128>(16 * pw + 4 * q + lg, 8 * m));
        if (WRITE_O)
#pragma unroll
            for (int q = 0; q < 2; ++q)  // token rows 32 pw + 16 q + m, columns 32 hb + 8 lg .. + 7
#pragma unroll
                for (int hb = 0; hb < NH; ++hb) {
                    const bf16x4_t lo = tr4<64>(sto, 32 * hb + 8 * lg, 32 * pw + 16 * q, lane);
                    const bf16x4_t hi = tr4<64>(sto, 32 * hb + 8 * lg + 4, 32 * pw + 16 * q, lane);
                    xo[q][hb] = bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                }
        if (STAGE_S) {
            uint16_t* gS = reinterpret_cast<uint16_t*>(slot(jc) + BwdExtra<128, true>::kS) + v0 * K;
#pragma unroll
            for (int q = 0; q < 4; ++q)
                *reinterpret_cast<bf16x8*>(gS + (16 * pw + 4 * q + lg) * K + 8 * m) = xs[q];
        }
        if (WRITE_O) {
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const int row = jc * kChunk + 32 * pw + 16 * q + m;
                if (row < len)
#pragma unroll
                    for (int hb = 0; hb < NH; ++hb)
                        *reinterpret_cast<bf16x8*>(og + ((start + row) * H + h) * V + v0 + 32 * hb + 8 * lg) =
                            xo[q][hb];
            }
        }
    };
    // ---- producer: one 4-byte copy per 128-byte line of chunk jc's operands,
    // all landing on the same 256 bytes of LDS
    auto warm = [&](int jc) {
        const uint8_t* base = slot(jc);
#pragma unroll
        for (int i = 0; i < NWARM; ++i) {
            int l = NVB * ((2 * i + pw) * 64 + lane) + vb;
            l = l < NL ? l : NL - 1;
            const uint8_t* a;
            if (l < NL_OP) a = base + (WRITE_O ? L::kQE : L::kW) + 128 * l;
            else if (WRITE_O && l < NL_OP + 64) a = base + L::kMS + 128 * (l - NL_OP);
            else if (l < NL - 4) a = base + L::kU + 128 * (l - (NL - 132));
            else a = base + L::kGC + 128 * (l - (NL - 4));
            __builtin_amdgcn_global_load_lds(a, (lds_void_t*)smj, 4, 0, 0);
        }
    };

    // ---- consumer: state strip, tile t = rows 16 t + 4 lg + r, column 16 w + m
    f32x4 S[8];
    // per-lane byte offsets of the operand fragments (loop invariant)
    int offA[4];      // [64][128] row fragment, k-step s, row tile 0 (+4096 per row tile)
    int offM[2];      // [64][64] row fragment, k-step s, row tile 0 (+2048 per row tile)
    int offT[8][2];   // [64][128] transposed fragment halves, column tile t, k-step 0 (+8192 per k-step)
#pragma unroll
    for (int s = 0; s < 4; ++s) offA[s] = swz_off<128>(m, 32 * s + 8 * lg);
#pragma unroll
    for (int s = 0; s < 2; ++s) offM[s] = swz_off<64>(m, 32 * s + 8 * lg);
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) offT[t][hh] = swz_off<128>(8 * lg + 4 * hh + (m >> 2), 16 * t + 4 * (m & 3));
    // At BV = 64 two waves share a SIMD, so a wave has 256 registers: column
    // tile t's offsets are formed from tile 0's (the tile index enters the
    // swizzled chunk index only through an exclusive or with 2 t), and the
    // decay factors are read a tile pair ahead instead of all at once.
    auto offTt = [&](int t, int hh) { return BV == 32 ? offT[t][hh] : (offT[0][hh] ^ (32 * t)); };
    // likewise the row fragments' k-steps (chunk index 4 s + lg)
    auto offAs = [&](int s) { return BV == 32 ? offA[s] : (offA[0] ^ (64 * s)); };
    auto offMs = [&](int s) { return BV == 32 ? offM[s] : (offM[0] ^ (64 * s)); };
    auto rdA = [](const uint8_t* tile, int off) { return *reinterpret_cast<const bf16x8*>(tile + off); };
    auto rdT = [](const uint8_t* tile, int off0, int off1) {
        const bf16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(tile + off0));
        const bf16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(tile + off1));
        return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    };
    auto step = [&](int jc) {
        const uint8_t* buf = smb + (jc & 1) * Z::kBuf;
        uint8_t* sts = sms + (jc & 1) * 8192;
        uint8_t* sto = smo + (jc & 1) * (128 * BV);
        bf16x8 Sb[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) Sb[s] = frag_acc_nat(S[2 * s], S[2 * s + 1]);
        // lane group lg of fragment s holds k = 32 s + 8 lg .. +7 of column 16 w + m
        if (STAGE_S) {  // S^T staging
#pragma unroll
            for (int s = 0; s < 4; ++s)
                *reinterpret_cast<bf16x8*>(sts + swz_off<128>(16 * w + m, 32 * s + 8 * lg)) = Sb[s];
        } else if (STORE) {  // straight to the slot's transposed entry state
            uint16_t* gS = reinterpret_cast<uint16_t*>(slot(jc) + BwdExtra<128, true>::kS) + (v0 + 16 * w + m) * K;
#pragma unroll
            for (int s = 0; s < 4; ++s) *reinterpret_cast<bf16x8*>(gS + 32 * s + 8 * lg) = Sb[s];
        }
        // The LDS reads are issued in batches ahead of the products that use
        // them (scheduling barriers keep that order), so that their latency
        // overlaps MFMA work rather than stalling each product.
        // W S and QE S for the strip's 64 x 16 block, one k-step of fragments ahead
        constexpr int NA = WRITE_O ? 8 : 4;
        bf16x8 fa[2][NA];
        auto load_a = [&](int s, bf16x8* f) {
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                f[rt] = rdA(buf + Z::oW + 4096 * rt, offAs(s));
                if (WRITE_O) f[4 + rt] = rdA(buf + Z::oQE + 4096 * rt, offAs(s));
            }
        };
        f32x4 ws_[4], o[4];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) ws_[rt] = o[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
        load_a(0, fa[0]);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            if (s < 3) load_a(s + 1, fa[(s + 1) & 1]);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                ws_[rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[s & 1][rt], Sb[s], ws_[rt], 0, 0, 0);
                if (WRITE_O)
                    o[rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[s & 1][4 + rt], Sb[s], o[rt], 0, 0, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        // operands of the remaining products: U rows, MS fragments, decay
        // factors, and the first KD^T fragments
        bf16x4_t u[4];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) u[rt] = tr4<BV>(buf + Z::oU, 16 * rt + 4 * lg, 16 * w, lane);
        bf16x8 fm[6];
        if (WRITE_O) {
#pragma unroll
            for (int rt = 0, q = 0; rt < 4; ++rt)
#pragma unroll
                for (int s = 0; s <= (rt >> 1); ++s, ++q) fm[q] = rdA(buf + Z::oMS + 2048 * rt, offMs(s));
        }
        f32x4 g[8];
        auto load_g = [&](int t) { g[t] = *reinterpret_cast<const f32x4*>(buf + Z::oGC + 4 * (16 * t + 4 * lg)); };
#pragma unroll
        for (int t = 0; t < (BV == 32 ? 8 : 2); ++t) load_g(t);
        bf16x8 fk[2][4];  // KD^T fragments of two column tiles, k-steps 0 and 1
        auto load_k = [&](int t, bf16x8* f) {
#pragma unroll
            for (int s = 0; s < 2; ++s) f[s] = rdT(buf + Z::oKD + 8192 * s, offTt(t, 0), offTt(t, 1));
        };
        load_k(0, &fk[0][0]);
        load_k(1, &fk[0][2]);
        __builtin_amdgcn_sched_barrier(0);
        // D = U - W S
        f32x4 d[4];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
#pragma unroll
            for (int r = 0; r < 4; ++r) d[rt][r] = static_cast<float>(u[rt][r]) - ws_[rt][r];
        const bf16x8 Db[2] = {frag_acc_nat(d[0], d[1]), frag_acc_nat(d[2], d[3])};
        // O = QE S + MS D (MS lower triangular)
        if (WRITE_O) {
#pragma unroll
            for (int rt = 0, q = 0; rt < 4; ++rt)
#pragma unroll
                for (int s = 0; s <= (rt >> 1); ++s, ++q)
                    o[rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fm[q], Db[s], o[rt], 0, 0, 0);
#pragma unroll
            for (int rt = 0; rt < 4; ++rt)
                *reinterpret_cast<bf16x4_t*>(sto + swz_off<64>(16 * w + m, 16 * rt + 4 * lg)) =
                    bf16x4_t{(__bf16)o[rt][0], (__bf16)o[rt][1], (__bf16)o[rt][2], (__bf16)o[rt][3]};
        }
        // S' = GC S + KD^T D, two column tiles at a time, the next two read ahead
#pragma unroll
        for (int tp = 0; tp < 4; ++tp) {
            if (tp < 3) {
                load_k(2 * tp + 2, &fk[(tp + 1) & 1][0]);
                load_k(2 * tp + 3, &fk[(tp + 1) & 1][2]);
                if (BV == 64) {
                    load_g(2 * tp + 2);
                    load_g(2 * tp + 3);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int t = 2 * tp + e;
#pragma unroll
                for (int r = 0; r < 4; ++r) S[t][r] *= g[t][r];
#pragma unroll
                for (int s = 0; s < 2; ++s)
                    S[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fk[tp & 1][2 * e + s], Db[s], S[t], 0, 0, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    if (prod) {
        if (nc > 0) fetch(0);
        wait_vmem_all();
    } else {
#pragma unroll
        for (int t = 0; t < 8; ++t) S[t] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (p.h0) {
#pragma unroll
            for (int t = 0; t < 8; ++t)
#pragma unroll
                for (int r = 0; r < 4; ++r) S[t][r] = p.h0[sbase + (16 * t + 4 * lg + r) * V + v0 + 16 * w + m];
        }
    }
    __syncthreads();
    // One loop per role (each wave passes the same nc barriers).  A shared
    // loop body makes the compiler keep both roles' values live at once
    // (288 registers against 194), and at BV = 64 it waited at the top of a
    // consumer's step for the producers' loads, and so for the consumer's own
    // state stores of the step before.
    if (prod) {
        for (int jc = 0; jc < nc; ++jc) {
            // staging reads before this step's copies (the compiler would wait
            // for the copies before any later LDS read); the warm-up loads are
            // issued last and are the only ones allowed to stay in flight
            if (jc > 0) drain(jc - 1);
            if (jc + 1 < nc) fetch(jc + 1);
            __builtin_amdgcn_sched_barrier(0);
            warm(jc + WA < nc ? jc + WA : jc);
            __builtin_amdgcn_sched_barrier(0);
            wait_vmem<NWARM>();
            barrier_lds();
        }
    } else {
        for (int jc = 0; jc < nc; ++jc) {
            step(jc);
            barrier_lds();
        }
    }
    if (prod) {
        if (nc > 0) drain(nc - 1);
    } else if (p.ht) {
#pragma unroll
        for (int t = 0; t < 8; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) p.ht[sbase + (16 * t + 4 * lg + r) * V + v0 + 16 * w + m] = S[t][r];
    }
}

// ------------------------------------------------------------------ state pass with the output gate
// Forward state pass for K = V = 128 in bf16 that applies the full-rank output
// gate of the "atlas_core/kimi_k3/kda.rs" page (full_rank_output_gate: per
// head, y = sigmoid(g) * o / sqrt(mean(o^2) + eps) over the head's V values) to
// every output row before it leaves the chip, so that o never makes a round
// trip through HBM.  The norm of a row needs all 128 value columns, so one
// workgroup owns a whole head (sequence, head): 4 waves, wave w the 32 value
// columns 32 w .. 32 w + 31 of the fp32 state (two 16-column strips over all
// 128 key rows, in MFMA accumulators, as the consumers of
// chunk_state_fwd_pc_kernel), so that every operand fragment read from LDS
// serves two strips.  There are no producer waves: each wave issues its share
// of the next chunk's direct global -> LDS copies (they hold no registers) at
// the start of a step and waits for them at its end, and requests the next
// chunk's gate inputs into registers.  Per chunk step:
//   O = QE S + MS D  (D = U - W S),  s_i = sum_v O_iv^2 over the four waves
//   (row sums in registers, exchanged through LDS), y = sigmoid(g) O / sqrt(s / 128 + eps),
//   S' = GC * S + KD^T D.
// Inference only: no entry state is stored for a backward.
struct StateGateFwd {
    static constexpr int oW = 0, oQE = 16384, oKD = 32768, oMS = 49152, oU = 57344, oGC = 73728;
    static constexpr int kBuf = 74240;  // one chunk's operand tiles (U: [64][128] swizzled)
};
constexpr int kGateStateThreads = 256;

template <bool GBF>  // gate input in bf16 (else fp32)
__global__ __launch_bounds__(kGateStateThreads) void chunk_state_fwd_gate_kernel(ChunkParams p,
                                                                                  const int32_t* chunk_off,
                                                                                  uint8_t* ws, int64_t slot_bytes) {
    using Z = StateGateFwd;
    using L = PrepLayout<128, true>;
    using GT = typename std::conditional<GBF, uint16_t, float>::type;
    constexpr int K = 128, V = 128, NWV = kGateStateThreads / 64;
    // 128-byte lines of one chunk's operands (QE, W, KD, MS, U, GC) warmed in
    // L2 kWarmAhead chunks ahead, NWARM loads per lane
    constexpr int NL = 384 + 64 + 128 + 4;
    constexpr int NWARM = (NL + kGateStateThreads - 1) / kGateStateThreads;
    __shared__ __attribute__((aligned(1024))) uint8_t smb[2 * Z::kBuf];
    __shared__ __attribute__((aligned(16))) float red[kChunk][NWV];  // per row: each wave's sum of squares
    __shared__ __attribute__((aligned(256))) uint8_t smj[256];

    const int chain = blockIdx.x;
    if (chain >= p.N * p.H) return;
    const int H = p.H;
    const int n = chain / H, h = chain % H;
    int64_t start;
    int len;
    seq_bounds(p, n, start, len);
    const int nc = chain_chunks(p, chunk_off, n, len);
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int lg = lane >> 4, m = lane & 15;
    const int64_t slot0 = chunk_slot(p, chunk_off, n, 0);
    const int64_t sbase = (static_cast<int64_t>(n) * H + h) * K * V;
    auto slot = [&](int jc) { return ws + ((slot0 + jc) * H + h) * slot_bytes; };
    const GT* gate = static_cast<const GT*>(p.out_gate);
    uint16_t* og = static_cast<uint16_t*>(p.o);
    // this lane's value columns: strip j of the wave, column 16 (2 w + j) + m

    // ---- this wave's share of chunk jc's direct copies into buffer jc & 1:
    // pieces w, w + 4, w + 8, w + 12 of W, KD, QE and U, pieces w and w + 4 of
    // MS, and (wave 0) GC
    auto fetch = [&](int jc) {
        const uint8_t* base = slot(jc);
        uint8_t* buf = smb + (jc & 1) * Z::kBuf;
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
            const int q = w + NWV * qq;
            dma_tile_piece<128>(reinterpret_cast<const uint16_t*>(base + L::kW), K, buf + Z::oW, q, lane);
            dma_tile_piece<128>(reinterpret_cast<const uint16_t*>(base + L::kKD), K, buf + Z::oKD, q, lane);
            dma_tile_piece<128>(reinterpret_cast<const uint16_t*>(base + L::kQE), K, buf + Z::oQE, q, lane);
            dma_tile_piece<128>(reinterpret_cast<const uint16_t*>(base + L::kU), V, buf + Z::oU, q, lane);
        }
#pragma unroll
        for (int qq = 0; qq < 2; ++qq)
            dma_tile_piece<64>(reinterpret_cast<const uint16_t*>(base + L::kMS), kChunk, buf + Z::oMS, w + NWV * qq,
                               lane);
        if (w == 0 && lane < 32) dma16(base + L::kGC + 16 * lane, buf + Z::oGC);
    };
    // ---- one 4-byte copy per 128-byte line of chunk jc's operands (L2 warm-up)
    auto warm = [&](int jc) {
        const uint8_t* base = slot(jc);
#pragma unroll
        for (int i = 0; i < NWARM; ++i) {
            int l = tid + kGateStateThreads * i;
            l = l < NL ? l : NL - 1;
            const uint8_t* a;
            if (l < 384) a = base + L::kQE + 128 * l;  // QE, W, KD are contiguous
            else if (l < 448) a = base + L::kMS + 128 * (l - 384);
            else if (l < 576) a = base + L::kU + 128 * (l - 448);
            else a = base + L::kGC + 128 * (l - 576);
            __builtin_amdgcn_global_load_lds(a, (lds_void_t*)smj, 4, 0, 0);
        }
    };
    // ---- chunk jc's gate inputs of this lane's 2 x 16 outputs (rows 16 rt +
    // 4 lg + r, strips j); rows past the end read the last row again (their
    // results are not stored)
    auto gload = [&](int jc, GT (&gr)[2][4][4]) {
        const int64_t row0 = start + static_cast<int64_t>(jc) * kChunk;
        const int rows = min(kChunk, len - jc * kChunk);
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = 16 * rt + 4 * lg + r;
                const int ic = i < rows ? i : rows - 1;
#pragma unroll
                for (int j = 0; j < 2; ++j) gr[j][rt][r] = gate[((row0 + ic) * H + h) * V + 16 * (2 * w + j) + m];
            }
    };

    // ---- state strips: tile t = key rows 16 t + 4 lg + r, column 16 (2 w + j) + m
    f32x4 S[2][8];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int t = 0; t < 8; ++t) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
                S[j][t][r] = p.h0 ? p.h0[sbase + (16 * t + 4 * lg + r) * V + 16 * (2 * w + j) + m] : 0.f;
        }
    auto rdA = [](const uint8_t* tile, int off) { return *reinterpret_cast<const bf16x8*>(tile + off); };
    auto rdT = [](const uint8_t* tile, int off0, int off1) {
        const bf16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(tile + off0));
        const bf16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(tile + off1));
        return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    };

    GT gcur[2][4][4];
    if (nc > 0) {
        gload(0, gcur);
        fetch(0);
    }
    wait_vmem_all();
    __syncthreads();
    for (int jc = 0; jc < nc; ++jc) {
        // per-lane LDS offsets from an opaque copy of the lane id, so that they
        // are recomputed per step rather than held in registers for the loop
        int ln = lane;
        asm volatile("" : "+v"(ln));
        const int mm = ln & 15, gg = ln >> 4;
        auto offA = [&](int s) { return swz_off<128>(mm, 32 * s + 8 * gg); };
        auto offM = [&](int s) { return swz_off<64>(mm, 32 * s + 8 * gg); };
        auto offT = [&](int t, int hh) { return swz_off<128>(8 * gg + 4 * hh + (mm >> 2), 16 * t + 4 * (mm & 3)); };
        const uint8_t* buf = smb + (jc & 1) * Z::kBuf;
        const int64_t row0 = start + static_cast<int64_t>(jc) * kChunk;
        const int rows = min(kChunk, len - jc * kChunk);
        // the next chunk's gate inputs and operand copies, and the L2 warm-up
        GT gnext[2][4][4];
        if (jc + 1 < nc) {
            gload(jc + 1, gnext);
            fetch(jc + 1);
        }
        warm(jc + kWarmAhead < nc ? jc + kWarmAhead : jc);
        __builtin_amdgcn_sched_barrier(0);

        // W S and QE S for both strips, one k-step of fragments ahead
        bf16x8 fa[2][8];
        auto load_a = [&](int s, bf16x8* f) {
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                f[rt] = rdA(buf + Z::oW + 4096 * rt, offA(s));
                f[4 + rt] = rdA(buf + Z::oQE + 4096 * rt, offA(s));
            }
        };
        f32x4 ws_[2][4], o[2][4];
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) ws_[j][rt] = o[j][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
        load_a(0, fa[0]);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            if (s < 3) load_a(s + 1, fa[(s + 1) & 1]);
            const bf16x8 Sb0 = frag_acc_nat(S[0][2 * s], S[0][2 * s + 1]);
            const bf16x8 Sb1 = frag_acc_nat(S[1][2 * s], S[1][2 * s + 1]);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                ws_[0][rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[s & 1][rt], Sb0, ws_[0][rt], 0, 0, 0);
                ws_[1][rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[s & 1][rt], Sb1, ws_[1][rt], 0, 0, 0);
                o[0][rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[s & 1][4 + rt], Sb0, o[0][rt], 0, 0, 0);
                o[1][rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[s & 1][4 + rt], Sb1, o[1][rt], 0, 0, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        // D = U - W S;  O += MS D (MS lower triangular)
        bf16x8 Db[2][2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            f32x4 d[4];
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                const bf16x4_t u = tr4<128>(buf + Z::oU, 16 * rt + 4 * gg, 16 * (2 * w + j), ln);
#pragma unroll
                for (int r = 0; r < 4; ++r) d[rt][r] = static_cast<float>(u[r]) - ws_[j][rt][r];
            }
            Db[j][0] = frag_acc_nat(d[0], d[1]);
            Db[j][1] = frag_acc_nat(d[2], d[3]);
        }
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
#pragma unroll
            for (int s = 0; s <= (rt >> 1); ++s) {
                const bf16x8 fm = rdA(buf + Z::oMS + 2048 * rt, offM(s));
                o[0][rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fm, Db[0][s], o[0][rt], 0, 0, 0);
                o[1][rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fm, Db[1][s], o[1][rt], 0, 0, 0);
            }
        // the rows' sums of squares over this wave's 32 columns; lane m records
        // row 16 (m / 4) + 4 lg + m % 4 of its lane group
        float mine = 0.f;
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float ss = row16_sum(o[0][rt][r] * o[0][rt][r] + o[1][rt][r] * o[1][rt][r]);
                mine = (m == 4 * rt + r) ? ss : mine;
            }
        red[16 * (m >> 2) + 4 * lg + (m & 3)][w] = mine;
        barrier_lds();  // every wave's sums are in red
        float rinv;
        {
            const float4 a4 = *reinterpret_cast<const float4*>(&red[16 * (m >> 2) + 4 * lg + (m & 3)][0]);
            rinv = rsqrtf(((a4.x + a4.y) + (a4.z + a4.w)) * (1.0f / V) + p.out_gate_eps);
        }
        uint16_t yv[2][4][4];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float ri = __shfl(rinv, 16 * lg + 4 * rt + r, 64);
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const float gi = GBF ? bf16_bits_to_f32(static_cast<uint16_t>(gcur[j][rt][r]))
                                         : static_cast<float>(gcur[j][rt][r]);
                    yv[j][rt][r] = f32_to_bf16_bits(sigmoidf_(gi) * o[j][rt][r] * ri);
                }
            }
        // S' = GC S + KD^T D: each KD^T fragment serves both strips
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const f32x4 g = *reinterpret_cast<const f32x4*>(buf + Z::oGC + 4 * (16 * t + 4 * gg));
            bf16x8 fk[2];
#pragma unroll
            for (int s = 0; s < 2; ++s) fk[s] = rdT(buf + Z::oKD + 8192 * s, offT(t, 0), offT(t, 1));
#pragma unroll
            for (int j = 0; j < 2; ++j) {
#pragma unroll
                for (int r = 0; r < 4; ++r) S[j][t][r] *= g[r];
#pragma unroll
                for (int s = 0; s < 2; ++s)
                    S[j][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fk[s], Db[j][s], S[j][t], 0, 0, 0);
            }
        }
        // this step's copies are done once at most its warm-up loads are
        // outstanding (one in-order counter: the next chunk's gate loads and
        // copies were issued before them); the row stores go out after that
        // wait, so that no step waits for a store
        wait_vmem<NWARM>();
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = 16 * rt + 4 * lg + r;
                if (i < rows) {
#pragma unroll
                    for (int j = 0; j < 2; ++j) og[((row0 + i) * H + h) * V + 16 * (2 * w + j) + m] = yv[j][rt][r];
                }
            }
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int rt = 0; rt < 4; ++rt)
#pragma unroll
                for (int r = 0; r < 4; ++r) gcur[j][rt][r] = gnext[j][rt][r];
        barrier_lds();
    }
    if (p.ht) {
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int t = 0; t < 8; ++t)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    p.ht[sbase + (16 * t + 4 * lg + r) * V + 16 * (2 * w + j) + m] = S[j][t][r];
    }
}

}  // namespace kda
