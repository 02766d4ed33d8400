// kda_decode.hip -- one decode token per sequence: short-conv update + one
// recurrence step, streaming the fp32 state once in and once out.
//
// Follows "atlas_core/kimi_k3/kda.rs" (Kimi K3 KDA CPU reference page):
// kda_decode_token runs conv_update over the 3*H*D [q|k|v] channels (window
// shifted left, newest sample in the last slot, SiLU of the kernel dot) and
// then kda_recurrent_step (L2-normalised q and k, sigmoid of the beta logit,
// key-axis decay, delta-rule write, read-out after the write).
//
// With a slot map, sequence n reads and writes the states of slot
// state_slots[n] of the state pools, so that a batch can resume sequences
// from saved snapshots (the prefix-hit restore that the same page's test
// prefix_hit_wrong_slot_diverges exercises); x, g, beta, o and the gate input
// stay indexed by n.
//
// Mapping: one workgroup per (sequence, head), 512 threads at D = 128 (256
// below; measured faster than 256 or 1024 at the production geometry).  The
// D x D state tile (64 KiB at D = 128) is held in registers: thread t owns column quad
// t % (D/4) and rows rg, rg + RG, rg + 2 RG, ... with rg = t / (D/4), so each
// load instruction of a wavefront covers whole 512-byte rows.  Every term of
// the step is local to a value column, so the only cross-thread traffic is
// two column reductions (S~^T k and S~^T q) through LDS.
//
// Bytes per (sequence, head) at D = 128, W = 4: state 2 x 64 KiB, conv state
// 2 x 6 KiB, x 768 B (bf16), g 512 B, conv_w 6 KiB (shared by all sequences),
// o 512 B, beta 4 B, and with the output gate its input, 256 B (bf16).
#include "kda_device.hpp"
#include "kda_launch.hpp"

namespace kda {

template <int D>
constexpr int decode_threads() { return D >= 128 ? 512 : 256; }

template <int D, typename XT>
__global__ __launch_bounds__(decode_threads<D>()) void decode_step_kernel(DecodeParams p) {
    constexpr int NT = decode_threads<D>();
    constexpr int CQ = D / 4;        // column quads
    constexpr int RG = NT / CQ;      // row groups
    constexpr int RPT = D / RG;      // rows per thread
    static_assert(CQ * RG == NT && RG * RPT == D, "tile shape");

    const int h = blockIdx.x;
    const int n = blockIdx.y;
    const int t = threadIdx.x;
    const int H = p.H;
    const int W = p.W;
    const int64_t HD = static_cast<int64_t>(H) * D;
    const int64_t CH = 3 * HD;

    __shared__ float ys[3][D];        // post-conv q | k | v of this head
    __shared__ float decay[D];        // exp(g_eff) per key row
    __shared__ float red_p[RG][D];    // partial S~^T k
    __shared__ float red_q[RG][D];    // partial S~^T q
    __shared__ float delta[D];
    __shared__ float scal[4];         // 1/|q|, 1/|k|, q^.k^
    __shared__ float osq[(D + kWave - 1) / kWave];  // per-wave sums of o^2 (output gate)

    // The sequence's states live in slot sn of the state pools (slot n
    // without a slot map).  A slot outside the pool leaves every state alone
    // and writes NaN outputs, so the error is visible.
    int sn = n;
    if (p.state_slots) {
        sn = p.state_slots[n];
        if (sn < 0 || sn >= p.n_slots) {
            for (int c = t; c < D; c += NT)
                p.o[static_cast<int64_t>(n) * HD + static_cast<int64_t>(h) * D + c] = __builtin_nanf("");
            return;
        }
    }

    // ---- issue the state loads first: they do not depend on the conv.
    float* Sg = p.state + (static_cast<int64_t>(sn) * H + h) * D * D;
    const int cq = t % CQ;
    const int rg = t / CQ;
    f32x4 s[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int r = rg + RG * i;
        s[i] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(Sg + r * D + 4 * cq));
    }

    // ---- short conv over this head's q, k, v channels
    const XT* x = static_cast<const XT*>(p.x) + static_cast<int64_t>(n) * CH;
    for (int j = t; j < 3 * D; j += NT) {
        const int part = j / D;
        const int c = j % D;
        const int64_t ch = part * HD + static_cast<int64_t>(h) * D + c;
        float* win = p.conv_state + (static_cast<int64_t>(sn) * CH + ch) * W;
        const float* w = p.conv_w + ch * W;
        const float xin = Elem<XT>::load(x, ch);
        float acc;
        if (W == 4) {
            f32x4 cw = *reinterpret_cast<const f32x4*>(win);
            f32x4 ww = *reinterpret_cast<const f32x4*>(w);
            f32x4 nw = {cw[1], cw[2], cw[3], xin};
            *reinterpret_cast<f32x4*>(win) = nw;
            acc = ww[0] * nw[0] + ww[1] * nw[1] + ww[2] * nw[2] + ww[3] * nw[3];
        } else {
            acc = 0.0f;
            for (int m = 0; m + 1 < W; ++m) {
                const float sh = win[m + 1];
                win[m] = sh;
                acc += w[m] * sh;
            }
            win[W - 1] = xin;
            acc += w[W - 1] * xin;
        }
        ys[part][c] = acc * sigmoidf_(acc);  // SiLU
    }

    // ---- gate (per key row)
    {
        const float rate = (p.gate_mode == GATE_LOGDECAY) ? 0.0f : __expf(p.A_log[h]);
        for (int c = t; c < D; c += NT) {
            const float gx = p.g[static_cast<int64_t>(n) * HD + static_cast<int64_t>(h) * D + c];
            const float bias = p.dt_bias ? p.dt_bias[static_cast<int64_t>(h) * D + c] : 0.0f;
            decay[c] = __expf(gate_eff(p.gate_mode, gx, rate, bias, p.lower_bound));
        }
    }
    __syncthreads();

    // ---- L2 norms and q^.k^ (wave 0: |q|^2, wave 1: |k|^2, wave 2: q.k)
    {
        const int wv = t / kWave, ln = t % kWave;
        if (wv < 3) {
            float acc = 0.0f;
            for (int c = ln; c < D; c += kWave) {
                const float a = (wv == 1) ? ys[1][c] : ys[0][c];
                const float b = (wv == 0) ? ys[0][c] : ys[1][c];
                acc += a * b;
            }
            acc = wave_sum(acc);
            if (ln == 0) scal[wv] = acc;
        }
    }
    __syncthreads();
    float rq = 1.0f, rk = 1.0f;
    if (p.use_qk_l2norm) {
        rq = rsqrtf(scal[0] + kL2Eps);
        rk = rsqrtf(scal[1] + kL2Eps);
    }
    const float kq = scal[2] * rq * rk;
    float braw = p.beta[static_cast<int64_t>(n) * H + h];
    const float beta = p.use_beta_sigmoid ? sigmoidf_(braw) : braw;

    // ---- decay rows, partial column sums of S~^T k and S~^T q
    f32x4 pk = {0.f, 0.f, 0.f, 0.f}, pq = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int r = rg + RG * i;
        const float e = decay[r];
        const float kr = ys[1][r] * rk;
        const float qr = ys[0][r] * rq;
        s[i] *= e;
        pk += s[i] * kr;
        pq += s[i] * qr;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        red_p[rg][4 * cq + j] = pk[j];
        red_q[rg][4 * cq + j] = pq[j];
    }
    __syncthreads();
    const int64_t oi = static_cast<int64_t>(n) * HD + static_cast<int64_t>(h) * D + t;
    const XT* og = static_cast<const XT*>(p.out_gate);
    float ov = 0.0f, gv = 0.0f;
    if (t < D) {
        if (og) gv = Elem<XT>::load(og, oi);
        float a = 0.0f, b = 0.0f;
#pragma unroll
        for (int g = 0; g < RG; ++g) {
            a += red_p[g][t];
            b += red_q[g][t];
        }
        const float d = beta * (ys[2][t] - a);
        delta[t] = d;
        ov = p.scale * (b + kq * d);
        if (!og) p.o[oi] = ov;
    }
    // full-rank output gate of the same page: sigmoid(g) * o / sqrt(mean(o^2) + eps)
    // over the head's D outputs, which are the first D threads
    if (og && t / kWave < (D + kWave - 1) / kWave) {
        const float s2 = wave_sum(ov * ov);  // threads t >= D hold 0
        if (t % kWave == 0) osq[t / kWave] = s2;
    }
    __syncthreads();
    if (og && t < D) {
        float ss = 0.0f;
#pragma unroll
        for (int w = 0; w < (D + kWave - 1) / kWave; ++w) ss += osq[w];
        p.o[oi] = sigmoidf_(gv) * ov * rsqrtf(ss * (1.0f / D) + p.out_gate_eps);
    }

    // ---- rank-1 write and store
    const f32x4 dq = *reinterpret_cast<const f32x4*>(&delta[4 * cq]);
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int r = rg + RG * i;
        const float kr = ys[1][r] * rk;
        s[i] += kr * dq;
        __builtin_nontemporal_store(s[i], reinterpret_cast<f32x4*>(Sg + r * D + 4 * cq));
    }
}

template <int D>
static hipError_t launch_decode_d(const DecodeParams& p, hipStream_t st) {
    dim3 grid(p.H, p.N);
    if (p.x_bf16)
        hipLaunchKernelGGL((decode_step_kernel<D, uint16_t>), grid, dim3(decode_threads<D>()), 0, st, p);
    else
        hipLaunchKernelGGL((decode_step_kernel<D, float>), grid, dim3(decode_threads<D>()), 0, st, p);
    return hipGetLastError();
}

hipError_t launch_decode(const DecodeParams& p, hipStream_t st) {
    switch (p.D) {
        case 32: return launch_decode_d<32>(p, st);
        case 64: return launch_decode_d<64>(p, st);
        case 128: return launch_decode_d<128>(p, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace kda
