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
// reads and writes whole contiguous row segments.  A second kernel writes the
// new conv state once every block has read the old one.
//
// Bytes per row and channel: x in, y out (its dtype each), plus (W-1)/64 of x
// re-read at block starts; conv_w and the states are per sequence.
#include "kda_device.hpp"
#include "kda_launch.hpp"

namespace kda {

typedef uint16_t u16x4_ __attribute__((ext_vector_type(4)));

constexpr int kConvRows = 64;     // rows per block
constexpr int kConvThreads = 256;
constexpr int kConvMaxW = 8;

template <typename T> struct Vec4;
template <> struct Vec4<float> {
    __device__ __forceinline__ static f32x4 load(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
    __device__ __forceinline__ static void store(float* p, f32x4 v) { *reinterpret_cast<f32x4*>(p) = v; }
};
template <> struct Vec4<uint16_t> {
    __device__ __forceinline__ static f32x4 load(const uint16_t* p) {
        const u16x4_ u = *reinterpret_cast<const u16x4_*>(p);
        return f32x4{bf16_bits_to_f32(u[0]), bf16_bits_to_f32(u[1]), bf16_bits_to_f32(u[2]), bf16_bits_to_f32(u[3])};
    }
    __device__ __forceinline__ static void store(uint16_t* p, f32x4 v) {
        const u16x4_ u = {f32_to_bf16_bits(v[0]), f32_to_bf16_bits(v[1]), f32_to_bf16_bits(v[2]), f32_to_bf16_bits(v[3])};
        *reinterpret_cast<u16x4_*>(p) = u;
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

template <typename XT, typename YT>
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

    f32x4 w[kConvMaxW];  // w[k][e]: weight of window slot k for channel c0 + e
#pragma unroll
    for (int k = 0; k < kConvMaxW; ++k)
        if (k < W)
#pragma unroll
            for (int e = 0; e < 4; ++e) w[k][e] = p.conv_w[(c0 + e) * W + k];

    // window slots 0 .. W-2 hold the inputs at rows r0 - (W-1) .. r0 - 1
    const int r0 = j * kConvRows;
    f32x4 win[kConvMaxW];
#pragma unroll
    for (int k = 0; k < kConvMaxW - 1; ++k) {
        if (k < W - 1) {
            const int tau = r0 - (W - 1) + k;
            if (tau >= 0) {
                win[k] = Vec4<XT>::load(x + (start + tau) * C + c0);
            } else if (p.conv_state) {
                // time tau < 0 sits in slot W + tau of the sequence's state
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    win[k][e] = p.conv_state[(static_cast<int64_t>(n) * C + c0 + e) * W + W + tau];
            } else {
                win[k] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
        }
    }

    const int part = static_cast<int>(c0 / HD);  // 0 q, 1 k, 2 v
    YT* dst = static_cast<YT*>(part == 0 ? p.q : (part == 1 ? p.k : p.v)) + (c0 - part * HD);
    const int r1 = min(len, r0 + kConvRows);
    for (int r = r0; r < r1; ++r) {
        win[W - 1] = Vec4<XT>::load(x + (start + r) * C + c0);
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k = 0; k < kConvMaxW; ++k)
            if (k < W)
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[e] += w[k][e] * win[k][e];
        f32x4 y;
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] = acc[e] * sigmoidf_(acc[e]);
        Vec4<YT>::store(dst + (start + r) * HD, y);
#pragma unroll
        for (int k = 0; k < kConvMaxW - 1; ++k)
            if (k < W - 1) win[k] = win[k + 1];
    }
}

// New conv state per (sequence, channel): slot k holds the input at time
// len - W + k, taken from the old state when that time is before the first row.
template <typename XT>
__global__ __launch_bounds__(kConvThreads) void conv_state_kernel(ConvParams p) {
    const int64_t C = 3 * static_cast<int64_t>(p.H) * p.D;
    const int64_t c = static_cast<int64_t>(blockIdx.x) * kConvThreads + threadIdx.x;
    const int n = blockIdx.y;
    if (c >= C) return;
    int64_t start;
    int len;
    if (p.cu_seqlens) {
        int a = p.cu_seqlens[n], b = p.cu_seqlens[n + 1];
        a = a < 0 ? 0 : (a > p.T ? p.T : a);
        b = b < a ? a : (b > p.T ? p.T : b);
        start = a;
        len = b - a;
    } else {
        start = static_cast<int64_t>(n) * p.T;
        len = p.T;
    }
    const XT* x = static_cast<const XT*>(p.x);
    const int W = p.W;
    float* st = p.conv_state + (static_cast<int64_t>(n) * C + c) * W;
    float nw[kConvMaxW];  // every old slot is read before any is written
#pragma unroll
    for (int k = 0; k < kConvMaxW; ++k)
        if (k < W) {
            const int tau = len - W + k;
            nw[k] = tau >= 0 ? Elem<XT>::load(x, (start + tau) * C + c) : st[W + tau];
        }
#pragma unroll
    for (int k = 0; k < kConvMaxW; ++k)
        if (k < W) st[k] = nw[k];
}

hipError_t launch_conv_prefill(const ConvParams& p, hipStream_t st) {
    const int64_t C = 3 * static_cast<int64_t>(p.H) * p.D;
    const unsigned gx = static_cast<unsigned>(p.block_bound);
    const unsigned gy = static_cast<unsigned>((C / 4 + kConvThreads - 1) / kConvThreads);
    if (gx > 0) {
        if (p.x_bf16 && p.y_bf16)
            hipLaunchKernelGGL((conv_prefill_kernel<uint16_t, uint16_t>), dim3(gx, gy), dim3(kConvThreads), 0, st, p);
        else if (p.x_bf16)
            hipLaunchKernelGGL((conv_prefill_kernel<uint16_t, float>), dim3(gx, gy), dim3(kConvThreads), 0, st, p);
        else if (p.y_bf16)
            hipLaunchKernelGGL((conv_prefill_kernel<float, uint16_t>), dim3(gx, gy), dim3(kConvThreads), 0, st, p);
        else
            hipLaunchKernelGGL((conv_prefill_kernel<float, float>), dim3(gx, gy), dim3(kConvThreads), 0, st, p);
    }
    if (p.conv_state && p.N > 0) {
        const unsigned sx = static_cast<unsigned>((C + kConvThreads - 1) / kConvThreads);
        if (p.x_bf16)
            hipLaunchKernelGGL((conv_state_kernel<uint16_t>), dim3(sx, p.N), dim3(kConvThreads), 0, st, p);
        else
            hipLaunchKernelGGL((conv_state_kernel<float>), dim3(sx, p.N), dim3(kConvThreads), 0, st, p);
    }
    return hipGetLastError();
}

}  // namespace kda
