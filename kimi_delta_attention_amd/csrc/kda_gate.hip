// kda_gate.hip -- the full-rank output gate and its reverse mode.
//
// Follows full_rank_output_gate of "atlas_core/kimi_k3/kda.rs" (Kimi K3 KDA
// CPU reference page): for every head of every row, with o the head's V
// output values and g its gate inputs,
//     r = 1 / sqrt(mean(o^2) + eps),   y = sigmoid(g) * o * r.
// The reverse mode is the chain rule written out, with a = sigmoid(g):
//     dg = dy * o * r * a (1 - a)
//     dO = r * a * dy - (r^3 / V) * o * sum(a * dy * o).
//
// Mapping: a head vector of V values is V/4 lanes of four consecutive values
// (8-byte bf16 or 16-byte fp32 vectors), so a wavefront reads whole
// contiguous rows; the row sums are xor-shuffle trees within those lanes.  A
// 256-thread workgroup takes kGateRounds groups of 256*4/V vectors, with
// every load of all its rounds issued before the first sum.  Loads past the
// last vector read the last vector again, and their results are not stored.
//
// Every value is read by the thread that writes the matching output, after
// all of its reads, so y may be o, dO may be dy, and dg may be g.
//
// Bytes per vector of V values: forward o and g in, y out; reverse o, g and
// dy in, dO and dg out (each in its own element type).
#include "kda_device.hpp"
#include "kda_launch.hpp"

namespace kda {

constexpr int kGateThreads = 256;
constexpr int kGateRounds = 4;

// Sum over the L lanes of one vector (L a power of two, groups aligned to L).
template <int L>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
    for (int m = L / 2; m > 0; m >>= 1) v += __shfl_xor(v, m, kWave);
    return v;
}

template <typename OT, typename GT, int V, bool BWD>
__global__ __launch_bounds__(kGateThreads) void output_gate_kernel(GateParams p) {
    constexpr int L = V / 4;                     // lanes per vector
    constexpr int PER_ROUND = kGateThreads / L;  // vectors per round
    static_assert(L >= 1 && L <= kWave && (L & (L - 1)) == 0, "V/4 lanes must divide a wavefront");
    const int64_t base = static_cast<int64_t>(blockIdx.x) * (kGateRounds * PER_ROUND) + threadIdx.x / L;
    const int q = threadIdx.x % L;
    const OT* o = static_cast<const OT*>(p.o);
    const GT* g = static_cast<const GT*>(p.g);
    const OT* dy = static_cast<const OT*>(p.dy);

    typename Vec4<OT>::Raw ro[kGateRounds], rd[kGateRounds];
    typename Vec4<GT>::Raw rg[kGateRounds];
    int64_t off[kGateRounds];
#pragma unroll
    for (int i = 0; i < kGateRounds; ++i) {
        int64_t vec = base + i * PER_ROUND;
        vec = vec < p.n_vec ? vec : p.n_vec - 1;
        off[i] = vec * V + 4 * q;
        ro[i] = Vec4<OT>::raw(o + off[i]);
        rg[i] = Vec4<GT>::raw(g + off[i]);
        if constexpr (BWD) rd[i] = Vec4<OT>::raw(dy + off[i]);
    }

    const float inv_v = 1.0f / V;
#pragma unroll
    for (int i = 0; i < kGateRounds; ++i) {
        const f32x4 ov = Vec4<OT>::cvt(ro[i]);
        const f32x4 gv = Vec4<GT>::cvt(rg[i]);
        f32x4 a;
#pragma unroll
        for (int e = 0; e < 4; ++e) a[e] = sigmoidf_(gv[e]);
        float ss = ov[0] * ov[0] + ov[1] * ov[1] + ov[2] * ov[2] + ov[3] * ov[3];
        const bool live = base + i * PER_ROUND < p.n_vec;
        if constexpr (!BWD) {
            ss = group_sum<L>(ss);
            const float r = rsqrtf(ss * inv_v + p.eps);
            f32x4 y;
#pragma unroll
            for (int e = 0; e < 4; ++e) y[e] = a[e] * ov[e] * r;
            if (live) Vec4<OT>::store(static_cast<OT*>(p.y) + off[i], y);
        } else {
            const f32x4 dv = Vec4<OT>::cvt(rd[i]);
            f32x4 ad;
#pragma unroll
            for (int e = 0; e < 4; ++e) ad[e] = a[e] * dv[e];
            float sa = ad[0] * ov[0] + ad[1] * ov[1] + ad[2] * ov[2] + ad[3] * ov[3];
            ss = group_sum<L>(ss);
            sa = group_sum<L>(sa);
            const float r = rsqrtf(ss * inv_v + p.eps);
            const float c = r * r * r * inv_v * sa;
            f32x4 dO, dg;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                dO[e] = r * ad[e] - c * ov[e];
                dg[e] = dv[e] * ov[e] * r * a[e] * (1.0f - a[e]);
            }
            if (live) {
                Vec4<OT>::store(static_cast<OT*>(p.dO) + off[i], dO);
                Vec4<GT>::store(static_cast<GT*>(p.dg) + off[i], dg);
            }
        }
    }
}

template <int V, bool BWD>
static void launch_gate_v(const GateParams& p, hipStream_t st) {
    constexpr int per_block = kGateRounds * (kGateThreads / (V / 4));
    const unsigned grid = static_cast<unsigned>((p.n_vec + per_block - 1) / per_block);
    if (p.o_bf16 && p.g_bf16)
        hipLaunchKernelGGL((output_gate_kernel<uint16_t, uint16_t, V, BWD>), dim3(grid), dim3(kGateThreads), 0, st, p);
    else if (p.o_bf16)
        hipLaunchKernelGGL((output_gate_kernel<uint16_t, float, V, BWD>), dim3(grid), dim3(kGateThreads), 0, st, p);
    else if (p.g_bf16)
        hipLaunchKernelGGL((output_gate_kernel<float, uint16_t, V, BWD>), dim3(grid), dim3(kGateThreads), 0, st, p);
    else
        hipLaunchKernelGGL((output_gate_kernel<float, float, V, BWD>), dim3(grid), dim3(kGateThreads), 0, st, p);
}

template <bool BWD>
static hipError_t launch_gate(const GateParams& p, hipStream_t st) {
    if (p.n_vec <= 0) return hipSuccess;
    switch (p.V) {
        case 32: launch_gate_v<32, BWD>(p, st); break;
        case 64: launch_gate_v<64, BWD>(p, st); break;
        case 128: launch_gate_v<128, BWD>(p, st); break;
        case 256: launch_gate_v<256, BWD>(p, st); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_output_gate(const GateParams& p, hipStream_t st) { return launch_gate<false>(p, st); }
hipError_t launch_output_gate_bwd(const GateParams& p, hipStream_t st) { return launch_gate<true>(p, st); }

}  // namespace kda
