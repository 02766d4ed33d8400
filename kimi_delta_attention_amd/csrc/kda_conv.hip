// kda_conv.hip -- stateful prefill of the short convolution: the conv_update of
// "atlas_core/kimi_k3/kda.rs" (Kimi K3 KDA CPU reference page: the window
// shifts left one slot, the new sample enters the last slot, and the output is
// the SiLU of the kernel dot) applied to every row of a sequence in order.  It
// starts from the sequence's conv state and leaves the window after its last
// row there, so that a prompt primed here continues exactly in the decode step
// ("memra-engine kda_fixture_gpu.rs" page, GATE 2 and GATE 3).
//
// Mapping: thread = 4 consecutive channels of one 64-row block of one
// sequence; workgroup = 256 threads (1024 channels).  Each thread reads the
// W-1 inputs before its block (from the rows before it, or from the conv
// state before the sequence's first row), then slides the window over its
// rows.  Rows are 16-byte (fp32) or 8-byte (bf16) vectors, so a wavefront
// reads and writes whole contiguous row segments.  A sequence's first block,
// the only one that reads the old conv state, also writes the new one.
//
// Bytes per row and channel: x in, y out (its dtype each), plus (W-1)/64 of x
// re-read at block starts; conv_w and the states are per sequence.
#include "kda_device.hpp"
#include "kda_launch.hpp"

namespace kda {

constexpr int kConvRows = kConvBlockRows;
constexpr int kConvGroup = 8;     // rows whose loads are issued together
constexpr int kConvThreads = 256;
constexpr int kConvMaxW = 8;
static_assert(kConvRows >= kConvMaxW - 1, "only a sequence's first block may read the old conv state");

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

template <typename XT, typename YT, int M>
__global__ __launch_bounds__(kConvThreads) void conv_prefill_kernel(ConvParams p) {
    const int64_t HD = static_cast<int64_t>(p.H) * p.D;
    const int64_t C = 3 * HD;
    const int64_t c0 = 4 * (static_cast<int64_t>(blockIdx.y) * kConvThreads + threadIdx.x);
    int n, j, len;
    int64_t start;
    if (!conv_block(p, blockIdx.x, n, j, start, len)) return;
    if (c0 >= C) return;
    const int W = p.W;
    const XT* x = static_cast<const XT*>(p.x);

    // A fixed window of M >= W slots, newest last, so that every register
    // index is static: slot s holds the input M-1-s rows back, and the W
    // weights sit in the last W slots (zeros before them).
    f32x4 w[M];  // w[s][e]: weight of slot s for channel c0 + e
    if (W == M) {
        // each channel's weights are M contiguous floats at a 16-byte boundary
        f32x4 cw[4][M / 4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
            for (int h = 0; h < M / 4; ++h)
                cw[e][h] = *reinterpret_cast<const f32x4*>(p.conv_w + (c0 + e) * M + 4 * h);
#pragma unroll
        for (int s = 0; s < M; ++s)
#pragma unroll
            for (int e = 0; e < 4; ++e) w[s][e] = cw[e][s / 4][s % 4];
    } else {
#pragma unroll
        for (int s = 0; s < M; ++s)
#pragma unroll
            for (int e = 0; e < 4; ++e) w[s][e] = s >= M - W ? p.conv_w[(c0 + e) * W + s - (M - W)] : 0.f;
    }

    const int part = static_cast<int>(c0 / HD);  // 0 q, 1 k, 2 v
    YT* dst = static_cast<YT*>(part == 0 ? p.q : (part == 1 ? p.k : p.v)) + (c0 - part * HD);
    const XT* xc = x + start * C + c0;  // this thread's channels at the sequence's row 0
    const int r0 = j * kConvRows;
    f32x4 win[M];

    // One row: the new input enters the last slot, the output is written and
    // the window shifts.
    auto row = [&](typename Vec4<XT>::Raw in, int r) {
        win[M - 1] = Vec4<XT>::cvt(in);
        f32x4 acc;
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] = w[0][e] * win[0][e];
#pragma unroll
        for (int s = 1; s < M; ++s)
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[e] += w[s][e] * win[s][e];
        f32x4 y;
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] = acc[e] * sigmoidf_(acc[e]);
        Vec4<YT>::store(dst + (start + r) * HD, y);
#pragma unroll
        for (int s = 0; s < M - 1; ++s) win[s] = win[s + 1];
    };

    if (r0 >= M - 1 && r0 + kConvRows <= len) {
        // A whole block with M-1 rows before it in the sequence: every load is
        // unconditional, and each group's loads are issued before the previous
        // group is computed, so the wait before a group's first use never
        // covers the stores just issued nor the next group's loads.
        typename Vec4<XT>::Raw xa[kConvGroup], xb[kConvGroup], xw[M - 1];
#pragma unroll
        for (int s = 0; s < M - 1; ++s) xw[s] = Vec4<XT>::raw(xc + static_cast<int64_t>(r0 - (M - 1) + s) * C);
#pragma unroll
        for (int i = 0; i < kConvGroup; ++i) xa[i] = Vec4<XT>::raw(xc + static_cast<int64_t>(r0 + i) * C);
#pragma unroll
        for (int s = 0; s < M - 1; ++s) win[s] = Vec4<XT>::cvt(xw[s]);
        constexpr int kGroups = kConvRows / kConvGroup;
        static_assert(kGroups % 2 == 0 && kGroups * kConvGroup == kConvRows, "groups are taken in pairs");
#pragma unroll
        for (int gi = 0; gi < kGroups; gi += 2) {
            const int ra = r0 + gi * kConvGroup, rb = ra + kConvGroup;
#pragma unroll
            for (int i = 0; i < kConvGroup; ++i) xb[i] = Vec4<XT>::raw(xc + static_cast<int64_t>(rb + i) * C);
#pragma unroll
            for (int i = 0; i < kConvGroup; ++i) row(xa[i], ra + i);
            if (gi + 2 < kGroups) {
#pragma unroll
                for (int i = 0; i < kConvGroup; ++i)
                    xa[i] = Vec4<XT>::raw(xc + static_cast<int64_t>(rb + kConvGroup + i) * C);
            }
#pragma unroll
            for (int i = 0; i < kConvGroup; ++i) row(xb[i], rb + i);
        }
        return;
    }

    // General block (a sequence's first rows, or its last partial block).
    // Slots 0 .. M-2 hold the inputs at rows r0 - (M-1) .. r0 - 1 (zero where
    // no weight reads them).
#pragma unroll
    for (int s = 0; s < M - 1; ++s) {
        const int tau = r0 - (M - 1) + s;
        win[s] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (s >= M - W) {
            if (tau >= 0) {
                win[s] = Vec4<XT>::load(xc + static_cast<int64_t>(tau) * C);
            } else if (p.conv_state) {
                // time tau < 0 sits in slot W + tau of the sequence's state
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    win[s][e] = p.conv_state[(static_cast<int64_t>(n) * C + c0 + e) * W + W + tau];
            }
        }
    }
    // rows in groups of kConvGroup, every load of a group issued before its first use
    const int r1 = min(len, r0 + kConvRows);
    for (int rb = r0; rb < r1; rb += kConvGroup) {
        typename Vec4<XT>::Raw xin[kConvGroup];
#pragma unroll
        for (int i = 0; i < kConvGroup; ++i)
            if (rb + i < r1) xin[i] = Vec4<XT>::raw(xc + static_cast<int64_t>(rb + i) * C);
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
        float* st = p.conv_state + (static_cast<int64_t>(n) * C + c0) * W;  // 4 channels x W slots
        float nw[4][kConvMaxW];
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
            for (int k = 0; k < kConvMaxW; ++k)
                if (k < W) {
                    const int tau = len - W + k;
                    nw[e][k] = tau >= 0 ? Elem<XT>::load(xc, static_cast<int64_t>(tau) * C + e) : st[e * W + W + tau];
                }
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
            for (int k = 0; k < kConvMaxW; ++k)
                if (k < W) st[e * W + k] = nw[e][k];
    }
}

hipError_t launch_conv_prefill(const ConvParams& p, hipStream_t st) {
    const int64_t C = 3 * static_cast<int64_t>(p.H) * p.D;
    const unsigned gx = static_cast<unsigned>(p.block_bound);
    const unsigned gy = static_cast<unsigned>((C / 4 + kConvThreads - 1) / kConvThreads);
    if (gx > 0) {
        const dim3 grid(gx, gy), block(kConvThreads);
        auto go = [&](auto kern) { hipLaunchKernelGGL(kern, grid, block, 0, st, p); };
        const bool w4 = p.W <= 4;
        if (p.x_bf16 && p.y_bf16)
            w4 ? go(conv_prefill_kernel<uint16_t, uint16_t, 4>) : go(conv_prefill_kernel<uint16_t, uint16_t, 8>);
        else if (p.x_bf16)
            w4 ? go(conv_prefill_kernel<uint16_t, float, 4>) : go(conv_prefill_kernel<uint16_t, float, 8>);
        else if (p.y_bf16)
            w4 ? go(conv_prefill_kernel<float, uint16_t, 4>) : go(conv_prefill_kernel<float, uint16_t, 8>);
        else
            w4 ? go(conv_prefill_kernel<float, float, 4>) : go(conv_prefill_kernel<float, float, 8>);
    }
    return hipGetLastError();
}

}  // namespace kda
