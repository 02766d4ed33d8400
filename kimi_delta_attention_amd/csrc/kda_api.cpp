// kda_api.cpp -- the C ABI declared in include/kda.h: host-side validation
// (nothing is launched on any error) and dispatch to the kernels.
#include <cmath>
#include <cstdint>

#include "kda.h"
#include "kda_launch.hpp"

namespace {

constexpr int kVersion = 1 * 10000 + 0 * 100 + 0;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool supported_dim(int d) { return d == 32 || d == 64 || d == 128; }

// eps of the gated output norm when the caller passes NaN: the value the
// "memra-engine kda_fixture_gpu.rs" page uses for it.
constexpr float kGateEpsDefault = 1e-5f;

// Shared validation of the chunk arguments; fills the internal launch params.
kda_status check_chunk(const kda_chunk_args* a, kda::ChunkParams& p, bool forward) {
    if (!a) return KDA_ERR_INVALID_ARG;
    if (a->B <= 0 || a->T < 0 || a->H <= 0 || a->K <= 0 || a->V <= 0) return KDA_ERR_INVALID_ARG;
    if (a->qkv_dtype != KDA_F32 && a->qkv_dtype != KDA_BF16) return KDA_ERR_UNSUPPORTED;
    if (a->chunk_size <= 0) return KDA_ERR_INVALID_ARG;  // a tiling request: the kernels tile with 64 rows
    // K = V in {32, 64, 128}, or the narrow-key pair K = 32, V = 64
    const bool kv_ok = (supported_dim(a->K) && a->K == a->V) || (a->K == 32 && a->V == 64);
    if (!kv_ok) return KDA_ERR_UNSUPPORTED;
    if (a->qkv_dtype == KDA_F32 && a->K > 64) return KDA_ERR_UNSUPPORTED;  // LDS budget
    if (a->gate_mode < KDA_GATE_LOGDECAY || a->gate_mode > KDA_GATE_SOFTPLUS) return KDA_ERR_INVALID_ARG;
    if (a->use_qk_l2norm != 0 && a->use_qk_l2norm != 1) return KDA_ERR_INVALID_ARG;
    if (a->use_beta_sigmoid != 0 && a->use_beta_sigmoid != 1) return KDA_ERR_INVALID_ARG;
    if (a->keep_for_backward != 0 && a->keep_for_backward != 1) return KDA_ERR_INVALID_ARG;
    int N = a->B;
    if (a->cu_seqlens) {
        if (a->B != 1 || a->N <= 0) return KDA_ERR_INVALID_ARG;
        N = a->N;
    }
    if (a->gate_mode != KDA_GATE_LOGDECAY && !a->A_log) return KDA_ERR_MISSING_PARAM;
    if (a->gate_mode == KDA_GATE_SAFE && std::isnan(a->lower_bound)) return KDA_ERR_MISSING_PARAM;
    const int64_t rows = static_cast<int64_t>(a->B) * a->T;
    if (rows > 0 && (!a->q || !a->k || !a->v || !a->g || !a->beta)) return KDA_ERR_INVALID_ARG;
    if (forward && rows > 0 && !a->o) return KDA_ERR_INVALID_ARG;
    if (forward && a->output_final_state && !a->final_state) return KDA_ERR_INVALID_ARG;
    const void* ptrs[] = {a->q, a->k, a->v, a->g, a->o, a->initial_state, a->final_state};
    for (const void* ptr : ptrs)
        if (ptr && !aligned16(ptr)) return KDA_ERR_INVALID_ARG;
    // element indices are formed in 64-bit; chunk counts and grid sizes in 32-bit
    if (rows * a->H > (int64_t(1) << 40)) return KDA_ERR_UNSUPPORTED;

    p.B = a->B; p.T = a->T; p.H = a->H; p.K = a->K; p.V = a->V;
    p.N = N;
    p.cu_seqlens = a->cu_seqlens;
    p.bf16 = a->qkv_dtype == KDA_BF16;
    p.q = a->q; p.k = a->k; p.v = a->v; p.g = a->g; p.beta = a->beta;
    p.A_log = a->A_log;
    p.dt_bias = a->dt_bias;
    p.scale = (std::isnan(a->scale) || a->scale <= 0.f) ? 1.0f / std::sqrt(static_cast<float>(a->K)) : a->scale;
    p.lower_bound = a->lower_bound;
    p.gate_mode = a->gate_mode;
    p.use_qk_l2norm = a->use_qk_l2norm;
    p.use_beta_sigmoid = a->use_beta_sigmoid;
    p.h0 = a->initial_state;
    p.o = forward ? a->o : nullptr;
    p.ht = (forward && a->output_final_state) ? a->final_state : nullptr;
    const int64_t nc_dense = (static_cast<int64_t>(a->T) + 63) / 64;
    const int64_t bound = a->cu_seqlens ? nc_dense + N : nc_dense * N;
    if (bound * a->H > INT32_MAX / 2) return KDA_ERR_UNSUPPORTED;
    p.keep = a->keep_for_backward != 0;
    if (a->out_gate) {
        // the fused output gate is an inference epilogue of the forward
        if (!forward || p.keep) return KDA_ERR_INVALID_ARG;
        if (a->out_gate_dtype != KDA_F32 && a->out_gate_dtype != KDA_BF16) return KDA_ERR_UNSUPPORTED;
        if (!(std::isnan(a->out_gate_eps) || a->out_gate_eps >= 0.f)) return KDA_ERR_INVALID_ARG;
        if (!aligned16(a->out_gate)) return KDA_ERR_INVALID_ARG;
        p.out_gate = a->out_gate;
        p.out_gate_bf16 = a->out_gate_dtype == KDA_BF16;
        p.out_gate_eps = std::isnan(a->out_gate_eps) ? kGateEpsDefault : a->out_gate_eps;
    }
    p.max_chunks = static_cast<int>(nc_dense);
    p.total_chunks_bound = static_cast<int>(bound);
    return KDA_OK;
}

}  // namespace

extern "C" {

const char* kda_status_string(kda_status s) {
    switch (s) {
        case KDA_OK: return "ok";
        case KDA_ERR_INVALID_ARG: return "invalid argument";
        case KDA_ERR_UNSUPPORTED: return "unsupported configuration";
        case KDA_ERR_MISSING_PARAM: return "missing gate parameter (A_log, or lower_bound for the safe gate)";
        case KDA_ERR_WORKSPACE: return "workspace missing or too small";
        case KDA_ERR_HIP: return "HIP launch error";
    }
    return "unknown status";
}

int kda_version(void) { return kVersion; }

size_t kda_chunk_fwd_workspace(const kda_chunk_args* a) {
    kda::ChunkParams p{};
    if (check_chunk(a, p, true) != KDA_OK) return 0;
    return p.keep ? kda::chunk_bwd_workspace(p) : kda::chunk_fwd_workspace(p);
}

static kda_status chunk_fwd_impl(const kda_chunk_args* a, int stage) {
    kda::ChunkParams p{};
    kda_status st = check_chunk(a, p, true);
    if (st != KDA_OK) return st;
    const size_t need = p.keep ? kda::chunk_bwd_workspace(p) : kda::chunk_fwd_workspace(p);
    if (need > 0 && (!a->workspace || a->workspace_bytes < need)) return KDA_ERR_WORKSPACE;
    if (a->workspace && !aligned16(a->workspace)) return KDA_ERR_WORKSPACE;
    hipError_t e = kda::launch_chunk_fwd(p, a->workspace, static_cast<hipStream_t>(a->stream), stage);
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

kda_status kda_chunk_fwd(const kda_chunk_args* a) { return chunk_fwd_impl(a, -1); }

static_assert(kda::kNoAllocScratchBytes == KDA_NOALLOC_SCRATCH_BYTES, "kda.h and the library agree on the size");

kda_status kda_chunk_fwd_noalloc(const kda_chunk_args* a) {
    kda::ChunkParams p{};
    kda_status st = check_chunk(a, p, true);
    if (st != KDA_OK) return st;
    if (p.keep) return KDA_ERR_INVALID_ARG;  // saved operands would not survive the next call
    const size_t need = kda::chunk_fwd_workspace(p);
    if (need > kda::kNoAllocScratchBytes) return KDA_ERR_WORKSPACE;
    void* ws = nullptr;
    if (need > 0 && kda::noalloc_workspace(&ws) != hipSuccess) return KDA_ERR_HIP;
    hipError_t e = kda::launch_chunk_fwd(p, ws, static_cast<hipStream_t>(a->stream), -1);
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

kda_status kda_chunk_fwd_stage(const kda_chunk_args* a, int stage) {
    if (stage < 0 || stage > 1) return KDA_ERR_INVALID_ARG;
    return chunk_fwd_impl(a, stage);
}

size_t kda_chunk_bwd_workspace(const kda_chunk_args* a) {
    kda::ChunkParams p{};
    if (check_chunk(a, p, false) != KDA_OK) return 0;
    return kda::chunk_bwd_workspace(p);
}

static kda_status chunk_bwd_impl(const kda_chunk_args* a, const kda_chunk_grads* gr, int stage) {
    kda::ChunkParams p{};
    kda_status st = check_chunk(a, p, false);
    if (st != KDA_OK) return st;
    if (!gr) return KDA_ERR_INVALID_ARG;
    const int64_t rows = static_cast<int64_t>(a->B) * a->T;
    if (rows > 0 && (!gr->dO || !gr->dq || !gr->dk || !gr->dv || !gr->dg || !gr->dbeta))
        return KDA_ERR_INVALID_ARG;
    const void* gptrs[] = {gr->dO, gr->d_final_state, gr->dq, gr->dk, gr->dv, gr->dg, gr->d_initial_state};
    for (const void* ptr : gptrs)
        if (ptr && !aligned16(ptr)) return KDA_ERR_INVALID_ARG;
    if (a->gate_mode == KDA_GATE_LOGDECAY && (gr->dA_log || gr->ddt_bias)) return KDA_ERR_INVALID_ARG;
    const size_t need = kda::chunk_bwd_workspace(p);
    if (need > 0 && (!a->workspace || a->workspace_bytes < need)) return KDA_ERR_WORKSPACE;
    if (a->workspace && !aligned16(a->workspace)) return KDA_ERR_WORKSPACE;
    kda::ChunkGrads g{};
    g.dO = gr->dO; g.dht = gr->d_final_state;
    g.dq = gr->dq; g.dk = gr->dk; g.dv = gr->dv; g.dg = gr->dg; g.dbeta = gr->dbeta;
    g.dh0 = gr->d_initial_state; g.dA_log = gr->dA_log; g.ddt_bias = gr->ddt_bias;
    hipError_t e = kda::launch_chunk_bwd(p, g, a->workspace, static_cast<hipStream_t>(a->stream), stage);
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

kda_status kda_chunk_bwd(const kda_chunk_args* a, const kda_chunk_grads* gr) { return chunk_bwd_impl(a, gr, -1); }

kda_status kda_chunk_bwd_stage(const kda_chunk_args* a, const kda_chunk_grads* gr, int stage) {
    if (stage < 0 || stage >= kda::kBwdStages) return KDA_ERR_INVALID_ARG;
    return chunk_bwd_impl(a, gr, stage);
}

int kda_chunk_bwd_stages(void) { return kda::kBwdStages; }

kda_status kda_recurrent_step(const kda_step_args* a) {
    if (!a) return KDA_ERR_INVALID_ARG;
    if (a->N < 0 || a->H <= 0 || a->D <= 0 || a->W < 1 || a->W > 8) return KDA_ERR_INVALID_ARG;
    if (!supported_dim(a->D)) return KDA_ERR_UNSUPPORTED;
    if (a->x_dtype != KDA_F32 && a->x_dtype != KDA_BF16) return KDA_ERR_UNSUPPORTED;
    if (a->gate_mode < KDA_GATE_LOGDECAY || a->gate_mode > KDA_GATE_SOFTPLUS) return KDA_ERR_INVALID_ARG;
    if (a->gate_mode != KDA_GATE_LOGDECAY && !a->A_log) return KDA_ERR_MISSING_PARAM;
    if (a->gate_mode == KDA_GATE_SAFE && std::isnan(a->lower_bound)) return KDA_ERR_MISSING_PARAM;
    if (a->N == 0) return KDA_OK;
    if (!a->x_qkv || !a->conv_w || !a->conv_state || !a->g || !a->beta || !a->state || !a->o)
        return KDA_ERR_INVALID_ARG;
    const void* sptrs[] = {a->conv_w, a->conv_state, a->state};
    for (const void* ptr : sptrs)
        if (!aligned16(ptr)) return KDA_ERR_INVALID_ARG;
    if (static_cast<int64_t>(a->N) > 65535) return KDA_ERR_UNSUPPORTED;  // grid y
    kda::DecodeParams p{};
    p.N = a->N; p.H = a->H; p.D = a->D; p.W = a->W;
    p.x_bf16 = a->x_dtype == KDA_BF16;
    p.x = a->x_qkv; p.conv_w = a->conv_w; p.conv_state = a->conv_state;
    p.g = a->g; p.beta = a->beta; p.A_log = a->A_log; p.dt_bias = a->dt_bias;
    p.lower_bound = a->lower_bound; p.gate_mode = a->gate_mode;
    p.use_qk_l2norm = a->use_qk_l2norm; p.use_beta_sigmoid = a->use_beta_sigmoid;
    p.scale = (std::isnan(a->scale) || a->scale <= 0.f) ? 1.0f / std::sqrt(static_cast<float>(a->D)) : a->scale;
    p.state = a->state; p.o = a->o;
    if (a->state_slots) {
        if (a->n_slots <= 0) return KDA_ERR_INVALID_ARG;
        p.state_slots = a->state_slots;
        p.n_slots = a->n_slots;
    }
    if (a->out_gate) {
        if (!(std::isnan(a->out_gate_eps) || a->out_gate_eps >= 0.f)) return KDA_ERR_INVALID_ARG;
        p.out_gate = a->out_gate;
        p.out_gate_eps = std::isnan(a->out_gate_eps) ? kGateEpsDefault : a->out_gate_eps;
    }
    hipError_t e = kda::launch_decode(p, static_cast<hipStream_t>(a->stream));
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

static kda_status check_gate(const kda_gate_args* a, kda::GateParams& p) {
    if (!a) return KDA_ERR_INVALID_ARG;
    if (a->rows < 0 || a->H <= 0 || a->V <= 0) return KDA_ERR_INVALID_ARG;
    if (a->V != 32 && a->V != 64 && a->V != 128 && a->V != 256) return KDA_ERR_UNSUPPORTED;
    if ((a->o_dtype != KDA_F32 && a->o_dtype != KDA_BF16) || (a->g_dtype != KDA_F32 && a->g_dtype != KDA_BF16))
        return KDA_ERR_UNSUPPORTED;
    if (!(std::isnan(a->eps) || a->eps >= 0.f)) return KDA_ERR_INVALID_ARG;
    p = kda::GateParams{};
    p.n_vec = static_cast<int64_t>(a->rows) * a->H;
    p.V = a->V;
    p.o_bf16 = a->o_dtype == KDA_BF16;
    p.g_bf16 = a->g_dtype == KDA_BF16;
    p.eps = std::isnan(a->eps) ? kGateEpsDefault : a->eps;
    p.o = a->o;
    p.g = a->g;
    if (p.n_vec * a->V > (int64_t(1) << 40)) return KDA_ERR_UNSUPPORTED;
    return KDA_OK;
}

kda_status kda_output_gate(const kda_gate_args* a) {
    kda::GateParams p;
    kda_status s = check_gate(a, p);
    if (s != KDA_OK) return s;
    if (p.n_vec == 0) return KDA_OK;
    if (!a->o || !a->g || !a->y) return KDA_ERR_INVALID_ARG;
    const void* ptrs[] = {a->o, a->g, a->y};
    for (const void* ptr : ptrs)
        if (!aligned16(ptr)) return KDA_ERR_INVALID_ARG;
    p.y = a->y;
    hipError_t e = kda::launch_output_gate(p, static_cast<hipStream_t>(a->stream));
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

kda_status kda_output_gate_bwd(const kda_gate_args* a, const void* dy, void* dO, void* dg) {
    kda::GateParams p;
    kda_status s = check_gate(a, p);
    if (s != KDA_OK) return s;
    if (p.n_vec == 0) return KDA_OK;
    if (!a->o || !a->g || !dy || !dO || !dg) return KDA_ERR_INVALID_ARG;
    const void* ptrs[] = {a->o, a->g, dy, dO, dg};
    for (const void* ptr : ptrs)
        if (!aligned16(ptr)) return KDA_ERR_INVALID_ARG;
    p.dy = dy;
    p.dO = dO;
    p.dg = dg;
    hipError_t e = kda::launch_output_gate_bwd(p, static_cast<hipStream_t>(a->stream));
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

kda_status kda_conv_prefill(const kda_conv_args* a) {
    if (!a) return KDA_ERR_INVALID_ARG;
    if (a->B <= 0 || a->T < 0 || a->H <= 0 || a->D <= 0 || a->W < 1 || a->W > 8) return KDA_ERR_INVALID_ARG;
    if (!supported_dim(a->D)) return KDA_ERR_UNSUPPORTED;
    if ((a->x_dtype != KDA_F32 && a->x_dtype != KDA_BF16) || (a->y_dtype != KDA_F32 && a->y_dtype != KDA_BF16))
        return KDA_ERR_UNSUPPORTED;
    int N = a->B;
    if (a->cu_seqlens) {
        if (a->B != 1 || a->N <= 0) return KDA_ERR_INVALID_ARG;
        N = a->N;
    }
    const int64_t rows = static_cast<int64_t>(a->B) * a->T;
    const int64_t C = 3 * static_cast<int64_t>(a->H) * a->D;
    if (!a->conv_w) return KDA_ERR_INVALID_ARG;
    if (rows > 0 && (!a->x_qkv || !a->q || !a->k || !a->v)) return KDA_ERR_INVALID_ARG;
    const void* ptrs[] = {a->x_qkv, a->conv_w, a->conv_state, a->q, a->k, a->v};
    for (const void* ptr : ptrs)
        if (ptr && !aligned16(ptr)) return KDA_ERR_INVALID_ARG;
    if (rows * C > (int64_t(1) << 40)) return KDA_ERR_UNSUPPORTED;
    const int64_t nb = (static_cast<int64_t>(a->T) + kda::kConvBlockRows - 1) / kda::kConvBlockRows;
    const int64_t block_bound = a->cu_seqlens ? nb + N : static_cast<int64_t>(N) * nb;
    if (block_bound * ((C / 4 + 255) / 256) > INT32_MAX || N > 65535) return KDA_ERR_UNSUPPORTED;
    // a block's rows are addressed by 32-bit byte offsets from its first input
    if (C * 4 * (kda::kConvBlockRows + 8) > INT32_MAX) return KDA_ERR_UNSUPPORTED;
    kda::ConvParams p{};
    p.B = a->B; p.T = a->T; p.H = a->H; p.D = a->D; p.W = a->W;
    p.N = N;
    p.cu_seqlens = a->cu_seqlens;
    p.x_bf16 = a->x_dtype == KDA_BF16;
    p.y_bf16 = a->y_dtype == KDA_BF16;
    p.x = a->x_qkv; p.conv_w = a->conv_w; p.conv_state = a->conv_state;
    p.q = a->q; p.k = a->k; p.v = a->v;
    p.block_bound = rows > 0 ? static_cast<int>(block_bound) : 0;
    hipError_t e = kda::launch_conv_prefill(p, static_cast<hipStream_t>(a->stream));
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

}  // extern "C"
