// kda_conv.hip -- stateful prefill of the short convolution: the conv_update of
// "atlas_core/kimi_k3/kda.rs" (Kimi K3 KDA CPU reference page: the window
// shifts left one slot, the new sample enters the last slot, and the output is
// the SiLU of the kernel dot) applied to every row of a sequence in order.  It
// starts from the sequence's conv state and leaves the window after its last
// row there, so that a prompt primed here continues exactly in the decode step
// ("memra-engine kda_fixture_gpu.rs" page, GATE 2 and GATE 3).
//
// Mapping: thread = 4 consecutive channels of one kConvBlockRows-row block of
// one sequence; workgroup = 256 threads (1024 channels); a one-dimensional grid
// with the channel slices of one block of rows next to each other.  Each
// thread reads the W-1 inputs before its block (from the rows before it, or
// from the conv state before the sequence's first row), then slides the window
// over its rows.  Rows are 16-byte (fp32) or 8-byte (bf16) vectors, so a
// wavefront reads and writes whole contiguous row segments.  A sequence's
// first block, the only one that reads the old conv state, also writes the
// new one.
//
// A whole block with W-1 rows before it reads its rows through a buffer
// resource based at the workgroup's first input, with the row offset in a
// scalar register, so that no vector instruction is spent on load addresses.
// Outputs are written with nontemporal stores.  The weights carry the factor
// -log2(e) of the SiLU's exponential: with a' = -log2(e) a,
// SiLU(a) = a / (1 + e^-a) = a' / ((1 + 2^a') (-log2(e))).
//
// Measured at 8192 rows x 6144 channels (bf16, cold caches): 16-row blocks
// beat 32 and 64 (more waves in flight per SIMD) and 8 (the halo re-read);
// 8 channels per thread, 4-row load groups, and giving each XCD a contiguous
// range of blocks were all slower.
//
// Bytes per row and channel: x in, y out (its dtype each), plus
// (W-1)/kConvBlockRows of x re-read at block starts; conv_w and the states
// are per sequence.
#include "kda_device.hpp"
#include "kda_launch.hpp"

namespace kda {

constexpr int kConvRows = kConvBlockRows;
constexpr int kConvThreads = 256;
constexpr int kConvCpt = 4;       // channels per thread
constexpr int kConvMaxW = 8;
static_assert(kConvRows >= kConvMaxW - 1, "only a sequence's first block may read the old conv state");
constexpr float kNegLog2e = -1.4426950408889634f;
constexpr int kBufferFlags = 0x00020000;  // word 3 of a gfx9 raw buffer resource

// SiLU of a from a' = -log2(e) a (see the header).
__device__ __forceinline__ float silu_scaled(float a2) {
    const float t = __builtin_amdgcn_exp2f(a2);
    return a2 * __builtin_amdgcn_rcpf(__builtin_fmaf(t, kNegLog2e, kNegLog2e));
}

// CPT consecutive channels of one row: Raw is the loaded form
// (kept until use), read through a pointer or a buffer resource (voff the
// lane's byte offset, soff the row's, wave-uniform).
template <typename T, int CPT> struct Row;
template <int CPT> struct Row<float, CPT> {
    struct Raw { f32x4 h[CPT / 4]; };
    __device__ __forceinline__ static Raw load(const float* p) {
        Raw r;
#pragma unroll
        for (int i = 0; i < CPT / 4; ++i) r.h[i] = *reinterpret_cast<const f32x4*>(p + 4 * i);
        return r;
    }
    __device__ __forceinline__ static Raw load(__amdgpu_buffer_rsrc_t rs, int voff, int soff) {
        Raw r;
#pragma unroll
        for (int i = 0; i < CPT / 4; ++i)
            r.h[i] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, voff + 16 * i, soff, 0));
        return r;
    }
    __device__ __forceinline__ static void cvt(const Raw& r, float (&x)[CPT]) {
#pragma unroll
        for (int e = 0; e < CPT; ++e) x[e] = r.h[e / 4][e % 4];
    }
    __device__ __forceinline__ static void store(float* p, const float (&x)[CPT]) {
#pragma unroll
        for (int i = 0; i < CPT / 4; ++i)
            __builtin_nontemporal_store(f32x4{x[4 * i], x[4 * i + 1], x[4 * i + 2], x[4 * i + 3]},
                                        reinterpret_cast<f32x4*>(p + 4 * i));
    }
};
template <> struct Row<uint16_t, 4> {
    using Raw = u16x4_;
    __device__ __forceinline__ static Raw load(const uint16_t* p) { return *reinterpret_cast<const u16x4_*>(p); }
    __device__ __forceinline__ static Raw load(__amdgpu_buffer_rsrc_t rs, int voff, int soff) {
        return __builtin_bit_cast(u16x4_, __builtin_amdgcn_raw_buffer_load_b64(rs, voff, soff, 0));
    }
    __device__ __forceinline__ static void cvt(const Raw& r, float (&x)[4]) {
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = bf16_bits_to_f32(r[e]);
    }
    __device__ __forceinline__ static void store(uint16_t* p, const float (&x)[4]) {
        __builtin_nontemporal_store(
            u16x4_{f32_to_bf16_bits(x[0]), f32_to_bf16_bits(x[1]), f32_to_bf16_bits(x[2]), f32_to_bf16_bits(x[3])},
            reinterpret_cast<u16x4_*>(p));
    }
};
// Sequence n and block j of row-block index s, walking the sequences' block
// counts; false when s is past the last block.
__device__ __forceinline__ bool conv_block(const ConvParams& p, int s, int& n, int& j, int64_t& start, int& len) {
    if (!p.cu_seqlens) {
        const int nb = (p.T + kConvRows - 1) / kConvRows;
        if (nb == 0) return false;
        n = s / nb;
        j = s % nb;
        start = static_cast<int64_t>(n) * p.T;
        len = p.T;
        return n < p.N;
    }
    int acc = 0;
    for (int q = 0; q < p.N; ++q) {
        int a = p.cu_seqlens[q], b = p.cu_seqlens[q + 1];
        a = a < 0 ? 0 : (a > p.T ? p.T : a);
        b = b < a ? a : (b > p.T ? p.T : b);
        const int nb = (b - a + kConvRows - 1) / kConvRows;
        if (s < acc + nb) {
            n = q;
            j = s - acc;
            start = a;
            len = b - a;
            return true;
        }
        acc += nb;
    }
    return false;
}

template <typename XT, typename YT, int M, int CPT>
__global__ __launch_bounds__(kConvThreads) void conv_prefill_kernel(ConvParams p) {
    constexpr int kSliceCh = CPT * kConvThreads;  // channels per workgroup
    const int64_t HD = static_cast<int64_t>(p.H) * p.D;
    const int64_t C = 3 * HD;
    // one-dimensional grid, channel slices fastest: the workgroups that cover
    // one block of rows are dispatched together and read whole rows between them
    const int slices = static_cast<int>((C + kSliceCh - 1) / kSliceCh);
    const int wg = static_cast<int>(blockIdx.x);
    const int slice = wg % slices;
    const int64_t c0 = static_cast<int64_t>(slice) * kSliceCh + CPT * threadIdx.x;
    int n, j, len;
    int64_t start;
    if (!conv_block(p, wg / slices, n, j, start, len)) return;
    if (c0 >= C) return;
    const int W = p.W;
    const XT* x = static_cast<const XT*>(p.x);
    using RX = Row<XT, CPT>;
    constexpr int kConvGroup = (32 / CPT < kConvRows / 2) ? 32 / CPT : kConvRows / 2;  // rows whose loads are issued together

    // A fixed window of M >= W slots, newest last, so that every register
    // index is static: slot s holds the input M-1-s rows back, and the W
    // weights sit in the last W slots (zeros before them).
    float w[M][CPT];  // w[s][e]: weight of slot s for channel c0 + e
    if (W == M) {
        // each channel's weights are M contiguous floats at a 16-byte boundary
#pragma unroll
        for (int e = 0; e < CPT; ++e)
#pragma unroll
            for (int h = 0; h < M / 4; ++h) {
                const f32x4 v = *reinterpret_cast<const f32x4*>(p.conv_w + (c0 + e) * M + 4 * h);
#pragma unroll
                for (int i = 0; i < 4; ++i) w[4 * h + i][e] = v[i];
            }
    } else {
#pragma unroll
        for (int s = 0; s < M; ++s)
#pragma unroll
            for (int e = 0; e < CPT; ++e) w[s][e] = s >= M - W ? p.conv_w[(c0 + e) * W + s - (M - W)] : 0.f;
    }
#pragma unroll
    for (int s = 0; s < M; ++s)
#pragma unroll
        for (int e = 0; e < CPT; ++e) w[s][e] *= kNegLog2e;

    const int part = static_cast<int>(c0 / HD);  // 0 q, 1 k, 2 v (HD is a multiple of CPT)
    YT* dst = static_cast<YT*>(part == 0 ? p.q : (part == 1 ? p.k : p.v)) + (c0 - part * HD);
    const XT* xc = x + start * C + c0;  // this thread's channels at the sequence's row 0
    const int r0 = j * kConvRows;
    float win[M][CPT];

    // One row: the new input enters the last slot, the output is written and
    // the window shifts.
    auto row = [&](const typename RX::Raw& in, int r) {
        RX::cvt(in, win[M - 1]);
        float y[CPT];
#pragma unroll
        for (int e = 0; e < CPT; ++e) {
            float acc = w[0][e] * win[0][e];
#pragma unroll
            for (int s = 1; s < M; ++s) acc += w[s][e] * win[s][e];
            y[e] = silu_scaled(acc);
        }
        Row<YT, CPT>::store(dst + (start + r) * HD, y);
#pragma unroll
        for (int s = 0; s < M - 1; ++s)
#pragma unroll
            for (int e = 0; e < CPT; ++e) win[s][e] = win[s + 1][e];
    };

    if (r0 >= M - 1 && r0 + kConvRows <= len) {
        // A whole block with M-1 rows before it in the sequence: every load is
        // unconditional, and each group's loads are issued before the previous
        // group is computed, so the wait before a group's first use never
        // covers the stores just issued nor the next group's loads.  Rows are
        // counted from the block's first input, M-1 rows before r0.
        const int64_t first = (start + r0 - (M - 1)) * C + static_cast<int64_t>(slice) * kSliceCh;
        const int64_t rows_all = p.cu_seqlens ? p.T : static_cast<int64_t>(p.N) * p.T;
        const int64_t extent = (rows_all * C - first) * static_cast<int64_t>(sizeof(XT));
        const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<XT*>(x + first), 0, static_cast<int>(extent < 0x7fffffff ? extent : 0x7fffffff), kBufferFlags);
        const int voff = threadIdx.x * CPT * static_cast<int>(sizeof(XT));
        const int rstride = static_cast<int>(C * sizeof(XT));
        typename RX::Raw xa[kConvGroup], xb[kConvGroup], xw[M - 1];
#pragma unroll
        for (int s = 0; s < M - 1; ++s) xw[s] = RX::load(rx, voff, s * rstride);
#pragma unroll
        for (int i = 0; i < kConvGroup; ++i) xa[i] = RX::load(rx, voff, (M - 1 + i) * rstride);
#pragma unroll
        for (int s = 0; s < M - 1; ++s) RX::cvt(xw[s], win[s]);
        constexpr int kGroups = kConvRows / kConvGroup;
        static_assert(kGroups % 2 == 0 && kGroups * kConvGroup == kConvRows, "groups are taken in pairs");
#pragma unroll
        for (int gi = 0; gi < kGroups; gi += 2) {
            const int ia = gi * kConvGroup, ib = ia + kConvGroup;  // rows after r0
#pragma unroll
            for (int i = 0; i < kConvGroup; ++i) xb[i] = RX::load(rx, voff, (M - 1 + ib + i) * rstride);
#pragma unroll
            for (int i = 0; i < kConvGroup; ++i) row(xa[i], r0 + ia + i);
            if (gi + 2 < kGroups) {
#pragma unroll
                for (int i = 0; i < kConvGroup; ++i)
                    xa[i] = RX::load(rx, voff, (M - 1 + ib + kConvGroup + i) * rstride);
            }
#pragma unroll
            for (int i = 0; i < kConvGroup; ++i) row(xb[i], r0 + ib + i);
        }
        return;
    }

    // General block (a sequence's first rows, or its last partial block).
    // Slots 0 .. M-2 hold the inputs at rows r0 - (M-1) .. r0 - 1 (zero where
    // no weight reads them).
#pragma unroll
    for (int s = 0; s < M - 1; ++s) {
        const int tau = r0 - (M - 1) + s;
#pragma unroll
        for (int e = 0; e < CPT; ++e) win[s][e] = 0.f;
        if (s >= M - W) {
            if (tau >= 0) {
                RX::cvt(RX::load(xc + static_cast<int64_t>(tau) * C), win[s]);
            } else if (p.conv_state) {
                // time tau < 0 sits in slot W + tau of the sequence's state
#pragma unroll
                for (int e = 0; e < CPT; ++e)
                    win[s][e] = p.conv_state[(static_cast<int64_t>(n) * C + c0 + e) * W + W + tau];
            }
        }
    }
    // rows in groups of kConvGroup, every load of a group issued before its first use
    const int r1 = min(len, r0 + kConvRows);
    for (int rb = r0; rb < r1; rb += kConvGroup) {
        typename RX::Raw xin[kConvGroup];
#pragma unroll
        for (int i = 0; i < kConvGroup; ++i)
            if (rb + i < r1) xin[i] = RX::load(xc + static_cast<int64_t>(rb + i) * C);
#pragma unroll
        for (int i = 0; i < kConvGroup; ++i) {
            if (rb + i >= r1) continue;  // (not break: the loop must unroll)
            row(xin[i], rb + i);
        }
    }

    if (j == 0 && p.conv_state) {
        // The sequence's first block is the only reader of the old state (later
        // blocks start at least kConvRows >= M - 1 rows in), so it writes the
        // new one, after its own reads: slot k takes the input at row
        // len - W + k, or the old slot W + (len - W + k) when that row is
        // before the first.
        float* st = p.conv_state + (static_cast<int64_t>(n) * C + c0) * W;  // CPT channels x W slots
        float nw[CPT][kConvMaxW];
#pragma unroll
        for (int e = 0; e < CPT; ++e)
#pragma unroll
            for (int k = 0; k < kConvMaxW; ++k)
                if (k < W) {
                    const int tau = len - W + k;
                    nw[e][k] = tau >= 0 ? Elem<XT>::load(xc, static_cast<int64_t>(tau) * C + e) : st[e * W + W + tau];
                }
#pragma unroll
        for (int e = 0; e < CPT; ++e)
#pragma unroll
            for (int k = 0; k < kConvMaxW; ++k)
                if (k < W) st[e * W + k] = nw[e][k];
    }
}

hipError_t launch_conv_prefill(const ConvParams& p, hipStream_t st) {
    const int64_t C = 3 * static_cast<int64_t>(p.H) * p.D;
    const int64_t slices = (C + kConvCpt * kConvThreads - 1) / (kConvCpt * kConvThreads);
    const unsigned gx = static_cast<unsigned>(p.block_bound * slices);
    auto go = [&](auto kern) {
        if (gx > 0) hipLaunchKernelGGL(kern, dim3(gx), dim3(kConvThreads), 0, st, p);
    };
#define KDA_CONV_GO(XT, YT, M) go(conv_prefill_kernel<XT, YT, M, kConvCpt>)
    const bool w4 = p.W <= 4;
    if (p.x_bf16 && p.y_bf16)
        w4 ? KDA_CONV_GO(uint16_t, uint16_t, 4) : KDA_CONV_GO(uint16_t, uint16_t, 8);
    else if (p.x_bf16)
        w4 ? KDA_CONV_GO(uint16_t, float, 4) : KDA_CONV_GO(uint16_t, float, 8);
    else if (p.y_bf16)
        w4 ? KDA_CONV_GO(float, uint16_t, 4) : KDA_CONV_GO(float, uint16_t, 8);
    else
        w4 ? KDA_CONV_GO(float, float, 4) : KDA_CONV_GO(float, float, 8);
#undef KDA_CONV_GO
    return hipGetLastError();
}

}  // namespace kda
