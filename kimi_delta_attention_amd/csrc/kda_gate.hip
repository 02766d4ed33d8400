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
// Mapping: a head vector of V values is V/8 lanes of eight consecutive values
// (16-byte bf16 vectors, or two 16-byte fp32 vectors), so a wavefront reads
// whole contiguous rows in 16-byte pieces; the row sums are xor-shuffle trees
// within those lanes.  A 256-thread workgroup takes kGateRounds groups of
// 256*8/V vectors, with every load of all its rounds issued before the first
// sum (one round is what the launch uses).  Loads past the last vector read the last vector again, and their
// results are not stored.
//
// Every value is read by the thread that writes the matching output, after
// all of its reads, so y may be o, dO may be dy, and dg may be g.
//
// Outputs are written with nontemporal stores (streaming data that no later
// read in the kernel wants cached); the reverse mode also reads its three
// inputs nontemporally.  Both choices were measured faster than plain
// accesses for their mode at 8192 x 16 x 128 bf16 with cold caches.
//
// Bytes per vector of V values: forward o and g in, y out; reverse o, g and
// dy in, dO and dg out (each in its own element type).
#include "kda_device.hpp"
#include "kda_launch.hpp"

namespace kda {

typedef uint16_t u16x8_t __attribute__((ext_vector_type(8)));

constexpr int kGateThreads = 256;
// One round per workgroup: at 8192 x 16 x 128 bf16 with cold caches the
// forward took 16.2-16.6 us with one round, 16.5 with two and 17.1 with four,
// the reverse mode 29.3, 30.6 and 31.4 us (more, smaller workgroups keep more
// requests in flight across the chip, as for a plain streaming copy).
constexpr int kGateRounds = 1;

// Sum over the L lanes of one vector (L a power of two, groups aligned to L).
template <int L>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
    for (int m = L / 2; m > 0; m >>= 1) v += __shfl_xor(v, m, kWave);
    return v;
}

// Eight consecutive elements: the loaded form (kept until use) and fp32.
template <typename T> struct Vec8;
template <> struct Vec8<float> {
    struct Raw { f32x4 a, b; };
    template <bool NT>
    __device__ __forceinline__ static Raw raw(const float* p) {
        if constexpr (NT)
            return Raw{__builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p)),
                       __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p + 4))};
        else
            return Raw{*reinterpret_cast<const f32x4*>(p), *reinterpret_cast<const f32x4*>(p + 4)};
    }
    __device__ __forceinline__ static void cvt(const Raw& r, float (&x)[8]) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            x[e] = r.a[e];
            x[4 + e] = r.b[e];
        }
    }
    __device__ __forceinline__ static void store(float* p, const float (&x)[8]) {
        __builtin_nontemporal_store(f32x4{x[0], x[1], x[2], x[3]}, reinterpret_cast<f32x4*>(p));
        __builtin_nontemporal_store(f32x4{x[4], x[5], x[6], x[7]}, reinterpret_cast<f32x4*>(p + 4));
    }
};
template <> struct Vec8<uint16_t> {  // bf16 bits
    using Raw = u16x8_t;
    template <bool NT>
    __device__ __forceinline__ static Raw raw(const uint16_t* p) {
        if constexpr (NT)
            return __builtin_nontemporal_load(reinterpret_cast<const u16x8_t*>(p));
        else
            return *reinterpret_cast<const u16x8_t*>(p);
    }
    __device__ __forceinline__ static void cvt(const Raw& r, float (&x)[8]) {
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = bf16_bits_to_f32(r[e]);
    }
    __device__ __forceinline__ static void store(uint16_t* p, const float (&x)[8]) {
        u16x8_t u;
#pragma unroll
        for (int e = 0; e < 8; ++e) u[e] = f32_to_bf16_bits(x[e]);
        __builtin_nontemporal_store(u, reinterpret_cast<u16x8_t*>(p));
    }
};

template <typename OT, typename GT, int V, bool BWD>
__global__ __launch_bounds__(kGateThreads) void output_gate_kernel(GateParams p) {
    constexpr int L = V / 8;                     // lanes per vector
    constexpr int PER_ROUND = kGateThreads / L;  // vectors per round
    static_assert(L >= 1 && L <= kWave && (L & (L - 1)) == 0, "V/8 lanes must divide a wavefront");
    const int64_t base = static_cast<int64_t>(blockIdx.x) * (kGateRounds * PER_ROUND) + threadIdx.x / L;
    const int q = threadIdx.x % L;
    const OT* o = static_cast<const OT*>(p.o);
    const GT* g = static_cast<const GT*>(p.g);
    const OT* dy = static_cast<const OT*>(p.dy);

    typename Vec8<OT>::Raw ro[kGateRounds], rd[kGateRounds];
    typename Vec8<GT>::Raw rg[kGateRounds];
    int64_t off[kGateRounds];
#pragma unroll
    for (int i = 0; i < kGateRounds; ++i) {
        int64_t vec = base + i * PER_ROUND;
        vec = vec < p.n_vec ? vec : p.n_vec - 1;
        off[i] = vec * V + 8 * q;
        ro[i] = Vec8<OT>::template raw<BWD>(o + off[i]);
        rg[i] = Vec8<GT>::template raw<BWD>(g + off[i]);
        if constexpr (BWD) rd[i] = Vec8<OT>::template raw<BWD>(dy + off[i]);
    }

    const float inv_v = 1.0f / V;
#pragma unroll
    for (int i = 0; i < kGateRounds; ++i) {
        float ov[8], gv[8], a[8];
        Vec8<OT>::cvt(ro[i], ov);
        Vec8<GT>::cvt(rg[i], gv);
        float ss = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            a[e] = sigmoidf_(gv[e]);
            ss += ov[e] * ov[e];
        }
        const bool live = base + i * PER_ROUND < p.n_vec;
        if constexpr (!BWD) {
            ss = group_sum<L>(ss);
            const float r = rsqrtf(ss * inv_v + p.eps);
            float y[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) y[e] = a[e] * ov[e] * r;
            if (live) Vec8<OT>::store(static_cast<OT*>(p.y) + off[i], y);
        } else {
            float dv[8], ad[8];
            Vec8<OT>::cvt(rd[i], dv);
            float sa = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                ad[e] = a[e] * dv[e];
                sa += ad[e] * ov[e];
            }
            ss = group_sum<L>(ss);
            sa = group_sum<L>(sa);
            const float r = rsqrtf(ss * inv_v + p.eps);
            const float c = r * r * r * inv_v * sa;
            float dO[8], dg[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                dO[e] = r * ad[e] - c * ov[e];
                dg[e] = dv[e] * ov[e] * r * a[e] * (1.0f - a[e]);
            }
            if (live) {
                Vec8<OT>::store(static_cast<OT*>(p.dO) + off[i], dO);
                Vec8<GT>::store(static_cast<GT*>(p.dg) + off[i], dg);
            }
        }
    }
}

template <int V, bool BWD>
static void launch_gate_v(const GateParams& p, hipStream_t st) {
    constexpr int per_block = kGateRounds * (kGateThreads / (V / 8));
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
