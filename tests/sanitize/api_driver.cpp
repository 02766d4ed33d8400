// Host-only driver of the C ABI's argument validation (kda_api.cpp), built
// with AddressSanitizer and UndefinedBehaviorSanitizer by
// tests/test_sanitizers.py.  The launch layer is replaced by stubs that only
// count calls, so every entry point runs its host checks without a GPU:
// valid calls must reach exactly one launch, invalid calls must return the
// documented status and launch nothing.  Exit status = number of failures.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "kda.h"
#include "kda_launch.hpp"

namespace kda {
static int g_launches = 0;
size_t chunk_fwd_workspace(const ChunkParams& p) {
    return 4096 + static_cast<size_t>(p.total_chunks_bound) * p.H * 1024;
}
size_t chunk_bwd_workspace(const ChunkParams& p) {
    return 4096 + static_cast<size_t>(p.total_chunks_bound) * p.H * 4096;
}
hipError_t launch_chunk_fwd(const ChunkParams& p, void*, hipStream_t, int) {
    ++g_launches;
    return (p.N >= 1 && p.max_chunks >= 0) ? hipSuccess : hipErrorInvalidValue;
}
hipError_t launch_chunk_bwd(const ChunkParams& p, const ChunkGrads&, void*, hipStream_t, int) {
    ++g_launches;
    return p.N >= 1 ? hipSuccess : hipErrorInvalidValue;
}
hipError_t launch_decode(const DecodeParams&, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_output_gate(const GateParams&, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_output_gate_bwd(const GateParams&, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_conv_prefill(const ConvParams&, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t noalloc_workspace(void** ptr) {
    *ptr = reinterpret_cast<void*>(uintptr_t(1) << 30);
    return hipSuccess;
}
}  // namespace kda

static int g_fail = 0;

// Never dereferenced: the stubs do not touch memory.
static void* fake(uintptr_t i) { return reinterpret_cast<void*>((uintptr_t(1) << 28) + 4096 * i); }

static void expect(const char* what, kda_status got, kda_status want, int launches_before, bool launch) {
    const int launched = kda::g_launches - launches_before;
    if (got != want || launched != (launch ? 1 : 0)) {
        std::printf("FAIL %s: status %d (want %d), launches %d\n", what, got, want, launched);
        ++g_fail;
    }
}

#define CHECK(what, call, want, launch)                     \
    do {                                                    \
        const int before_ = kda::g_launches;                \
        const kda_status st_ = (call);                      \
        expect(what, st_, want, before_, launch);           \
    } while (0)

static kda_chunk_args chunk_args() {
    kda_chunk_args a;
    std::memset(&a, 0, sizeof(a));
    a.B = 2; a.T = 130; a.H = 3; a.K = 128; a.V = 128;
    a.qkv_dtype = KDA_BF16;
    a.q = fake(1); a.k = fake(2); a.v = fake(3); a.g = static_cast<const float*>(fake(4));
    a.beta = static_cast<const float*>(fake(5));
    a.scale = NAN; a.lower_bound = NAN; a.chunk_size = 64;
    a.o = fake(6);
    a.workspace = fake(100);
    a.workspace_bytes = size_t(1) << 30;
    return a;
}

int main() {
    // ---- chunk forward
    kda_chunk_args a = chunk_args();
    CHECK("fwd valid", kda_chunk_fwd(&a), KDA_OK, true);
    CHECK("fwd null args", kda_chunk_fwd(nullptr), KDA_ERR_INVALID_ARG, false);
    { kda_chunk_args b = a; b.B = 0; CHECK("fwd B=0", kda_chunk_fwd(&b), KDA_ERR_INVALID_ARG, false); }
    { kda_chunk_args b = a; b.T = -1; CHECK("fwd T<0", kda_chunk_fwd(&b), KDA_ERR_INVALID_ARG, false); }
    { kda_chunk_args b = a; b.K = b.V = 48; CHECK("fwd K=48", kda_chunk_fwd(&b), KDA_ERR_UNSUPPORTED, false); }
    { kda_chunk_args b = a; b.V = 64; CHECK("fwd K128 V64", kda_chunk_fwd(&b), KDA_ERR_UNSUPPORTED, false); }
    { kda_chunk_args b = a; b.qkv_dtype = KDA_F32; CHECK("fwd fp32 K128", kda_chunk_fwd(&b), KDA_ERR_UNSUPPORTED, false); }
    { kda_chunk_args b = a; b.qkv_dtype = 7; CHECK("fwd dtype", kda_chunk_fwd(&b), KDA_ERR_UNSUPPORTED, false); }
    { kda_chunk_args b = a; b.gate_mode = 5; CHECK("fwd gate mode", kda_chunk_fwd(&b), KDA_ERR_INVALID_ARG, false); }
    { kda_chunk_args b = a; b.use_qk_l2norm = 2; CHECK("fwd l2 flag", kda_chunk_fwd(&b), KDA_ERR_INVALID_ARG, false); }
    { kda_chunk_args b = a; b.use_beta_sigmoid = -1; CHECK("fwd sigmoid flag", kda_chunk_fwd(&b), KDA_ERR_INVALID_ARG, false); }
    { kda_chunk_args b = a; b.keep_for_backward = 3; CHECK("fwd keep flag", kda_chunk_fwd(&b), KDA_ERR_INVALID_ARG, false); }
    { kda_chunk_args b = a; b.chunk_size = 0; CHECK("fwd chunk 0", kda_chunk_fwd(&b), KDA_ERR_INVALID_ARG, false); }
    { kda_chunk_args b = a; b.cu_seqlens = static_cast<const int32_t*>(fake(7)); b.N = 2;
      CHECK("fwd varlen B=2", kda_chunk_fwd(&b), KDA_ERR_INVALID_ARG, false);
      b.B = 1; b.N = 0; CHECK("fwd varlen N=0", kda_chunk_fwd(&b), KDA_ERR_INVALID_ARG, false);
      b.N = 3; CHECK("fwd varlen valid", kda_chunk_fwd(&b), KDA_OK, true); }
    { kda_chunk_args b = a; b.gate_mode = KDA_GATE_SOFTPLUS; CHECK("fwd softplus no A_log", kda_chunk_fwd(&b), KDA_ERR_MISSING_PARAM, false);
      b.A_log = static_cast<const float*>(fake(8)); CHECK("fwd softplus", kda_chunk_fwd(&b), KDA_OK, true);
      b.gate_mode = KDA_GATE_SAFE; CHECK("fwd safe no lb", kda_chunk_fwd(&b), KDA_ERR_MISSING_PARAM, false);
      b.lower_bound = -5.f; CHECK("fwd safe", kda_chunk_fwd(&b), KDA_OK, true); }
    { kda_chunk_args b = a; b.q = nullptr; CHECK("fwd null q", kda_chunk_fwd(&b), KDA_ERR_INVALID_ARG, false); }
    { kda_chunk_args b = a; b.o = nullptr; CHECK("fwd null o", kda_chunk_fwd(&b), KDA_ERR_INVALID_ARG, false); }
    { kda_chunk_args b = a; b.T = 0; b.q = b.k = b.v = nullptr; b.o = nullptr;
      CHECK("fwd empty", kda_chunk_fwd(&b), KDA_OK, true); }
    { kda_chunk_args b = a; b.k = static_cast<const char*>(b.k) + 2; CHECK("fwd misaligned k", kda_chunk_fwd(&b), KDA_ERR_INVALID_ARG, false); }
    { kda_chunk_args b = a; b.output_final_state = 1; CHECK("fwd final null", kda_chunk_fwd(&b), KDA_ERR_INVALID_ARG, false); }
    { kda_chunk_args b = a; b.workspace_bytes = 16; CHECK("fwd small ws", kda_chunk_fwd(&b), KDA_ERR_WORKSPACE, false); }
    { kda_chunk_args b = a; b.workspace = nullptr; CHECK("fwd null ws", kda_chunk_fwd(&b), KDA_ERR_WORKSPACE, false); }
    { kda_chunk_args b = a; b.workspace = static_cast<char*>(b.workspace) + 8; CHECK("fwd misaligned ws", kda_chunk_fwd(&b), KDA_ERR_WORKSPACE, false); }
    { kda_chunk_args b = a; b.B = 1 << 20; b.T = 1 << 20; CHECK("fwd too large", kda_chunk_fwd(&b), KDA_ERR_UNSUPPORTED, false); }
    { kda_chunk_args b = a; b.K = 32; b.V = 64; b.qkv_dtype = KDA_F32; CHECK("fwd narrow key fp32", kda_chunk_fwd(&b), KDA_OK, true); }
    CHECK("fwd stage 1", kda_chunk_fwd_stage(&a, 1), KDA_OK, true);
    CHECK("fwd stage 2", kda_chunk_fwd_stage(&a, 2), KDA_ERR_INVALID_ARG, false);
    if (kda_chunk_fwd_workspace(&a) == 0) { std::printf("FAIL fwd workspace query\n"); ++g_fail; }
    if (kda_chunk_fwd_workspace(nullptr) != 0) { std::printf("FAIL fwd workspace null\n"); ++g_fail; }
    // ---- the no-allocation forward
    CHECK("noalloc valid", kda_chunk_fwd_noalloc(&a), KDA_OK, true);
    { kda_chunk_args b = a; b.keep_for_backward = 1; CHECK("noalloc keep", kda_chunk_fwd_noalloc(&b), KDA_ERR_INVALID_ARG, false); }
    { kda_chunk_args b = a; b.T = 1 << 20; b.H = 64; CHECK("noalloc oversized", kda_chunk_fwd_noalloc(&b), KDA_ERR_WORKSPACE, false); }
    // ---- chunk backward
    kda_chunk_grads g;
    std::memset(&g, 0, sizeof(g));
    g.dO = fake(20); g.dq = fake(21); g.dk = fake(22); g.dv = fake(23);
    g.dg = static_cast<float*>(fake(24)); g.dbeta = static_cast<float*>(fake(25));
    CHECK("bwd valid", kda_chunk_bwd(&a, &g), KDA_OK, true);
    CHECK("bwd null grads", kda_chunk_bwd(&a, nullptr), KDA_ERR_INVALID_ARG, false);
    { kda_chunk_grads h = g; h.dO = nullptr; CHECK("bwd null dO", kda_chunk_bwd(&a, &h), KDA_ERR_INVALID_ARG, false); }
    { kda_chunk_grads h = g; h.dq = static_cast<char*>(h.dq) + 4; CHECK("bwd misaligned dq", kda_chunk_bwd(&a, &h), KDA_ERR_INVALID_ARG, false); }
    { kda_chunk_grads h = g; h.dA_log = static_cast<float*>(fake(26)); CHECK("bwd dA_log logdecay", kda_chunk_bwd(&a, &h), KDA_ERR_INVALID_ARG, false); }
    { kda_chunk_args b = a; b.workspace_bytes = 4096; CHECK("bwd small ws", kda_chunk_bwd(&b, &g), KDA_ERR_WORKSPACE, false); }
    CHECK("bwd stage 4", kda_chunk_bwd_stage(&a, &g, 4), KDA_OK, true);
    CHECK("bwd stage 5", kda_chunk_bwd_stage(&a, &g, kda_chunk_bwd_stages()), KDA_ERR_INVALID_ARG, false);
    // ---- decode
    kda_step_args d;
    std::memset(&d, 0, sizeof(d));
    d.N = 4; d.H = 2; d.D = 128; d.W = 4; d.x_dtype = KDA_BF16;
    d.x_qkv = fake(30); d.conv_w = static_cast<const float*>(fake(31)); d.conv_state = static_cast<float*>(fake(32));
    d.g = static_cast<const float*>(fake(33)); d.beta = static_cast<const float*>(fake(34));
    d.state = static_cast<float*>(fake(35)); d.o = static_cast<float*>(fake(36));
    d.lower_bound = NAN; d.scale = NAN; d.out_gate_eps = NAN;
    CHECK("decode valid", kda_recurrent_step(&d), KDA_OK, true);
    CHECK("decode null", kda_recurrent_step(nullptr), KDA_ERR_INVALID_ARG, false);
    { kda_step_args e = d; e.N = 0; CHECK("decode N=0", kda_recurrent_step(&e), KDA_OK, false); }
    { kda_step_args e = d; e.N = -1; CHECK("decode N<0", kda_recurrent_step(&e), KDA_ERR_INVALID_ARG, false); }
    { kda_step_args e = d; e.D = 48; CHECK("decode D=48", kda_recurrent_step(&e), KDA_ERR_UNSUPPORTED, false); }
    { kda_step_args e = d; e.W = 9; CHECK("decode W=9", kda_recurrent_step(&e), KDA_ERR_INVALID_ARG, false); }
    { kda_step_args e = d; e.state = nullptr; CHECK("decode null state", kda_recurrent_step(&e), KDA_ERR_INVALID_ARG, false); }
    { kda_step_args e = d; e.state = reinterpret_cast<float*>(reinterpret_cast<char*>(e.state) + 4);
      CHECK("decode misaligned state", kda_recurrent_step(&e), KDA_ERR_INVALID_ARG, false); }
    { kda_step_args e = d; e.gate_mode = KDA_GATE_SAFE; e.A_log = static_cast<const float*>(fake(37));
      CHECK("decode safe no lb", kda_recurrent_step(&e), KDA_ERR_MISSING_PARAM, false); }
    { kda_step_args e = d; e.state_slots = static_cast<const int32_t*>(fake(38));
      CHECK("decode slots n=0", kda_recurrent_step(&e), KDA_ERR_INVALID_ARG, false);
      e.n_slots = 9; CHECK("decode slots", kda_recurrent_step(&e), KDA_OK, true); }
    { kda_step_args e = d; e.out_gate = fake(39); e.out_gate_eps = -1.f;
      CHECK("decode gate eps<0", kda_recurrent_step(&e), KDA_ERR_INVALID_ARG, false); }
    { kda_step_args e = d; e.N = 70000; CHECK("decode N too large", kda_recurrent_step(&e), KDA_ERR_UNSUPPORTED, false); }
    // ---- conv prefill
    kda_conv_args c;
    std::memset(&c, 0, sizeof(c));
    c.B = 2; c.T = 100; c.H = 2; c.D = 64; c.W = 4; c.x_dtype = KDA_BF16; c.y_dtype = KDA_BF16;
    c.x_qkv = fake(40); c.conv_w = static_cast<const float*>(fake(41)); c.q = fake(42); c.k = fake(43); c.v = fake(44);
    CHECK("conv valid", kda_conv_prefill(&c), KDA_OK, true);
    { kda_conv_args e = c; e.D = 48; CHECK("conv D=48", kda_conv_prefill(&e), KDA_ERR_UNSUPPORTED, false); }
    { kda_conv_args e = c; e.W = 0; CHECK("conv W=0", kda_conv_prefill(&e), KDA_ERR_INVALID_ARG, false); }
    { kda_conv_args e = c; e.cu_seqlens = static_cast<const int32_t*>(fake(45)); e.N = 2;
      CHECK("conv varlen B=2", kda_conv_prefill(&e), KDA_ERR_INVALID_ARG, false); }
    { kda_conv_args e = c; e.conv_w = nullptr; CHECK("conv null w", kda_conv_prefill(&e), KDA_ERR_INVALID_ARG, false); }
    { kda_conv_args e = c; e.x_qkv = static_cast<const char*>(e.x_qkv) + 2; CHECK("conv misaligned x", kda_conv_prefill(&e), KDA_ERR_INVALID_ARG, false); }
    // ---- output gate
    kda_gate_args o;
    std::memset(&o, 0, sizeof(o));
    o.rows = 10; o.H = 2; o.V = 128; o.o_dtype = KDA_BF16; o.g_dtype = KDA_F32; o.eps = NAN;
    o.o = fake(50); o.g = fake(51); o.y = fake(52);
    CHECK("gate valid", kda_output_gate(&o), KDA_OK, true);
    { kda_gate_args e = o; e.V = 48; CHECK("gate V=48", kda_output_gate(&e), KDA_ERR_UNSUPPORTED, false); }
    { kda_gate_args e = o; e.eps = -1.f; CHECK("gate eps<0", kda_output_gate(&e), KDA_ERR_INVALID_ARG, false); }
    { kda_gate_args e = o; e.rows = 0; CHECK("gate empty", kda_output_gate(&e), KDA_OK, false); }
    { kda_gate_args e = o; e.y = nullptr; CHECK("gate null y", kda_output_gate(&e), KDA_ERR_INVALID_ARG, false); }
    CHECK("gate bwd valid", kda_output_gate_bwd(&o, fake(53), fake(54), fake(55)), KDA_OK, true);
    CHECK("gate bwd null dy", kda_output_gate_bwd(&o, nullptr, fake(54), fake(55)), KDA_ERR_INVALID_ARG, false);
    // ---- strings
    for (int s = -1; s <= 6; ++s)
        if (!kda_status_string(static_cast<kda_status>(s))) { std::printf("FAIL status string %d\n", s); ++g_fail; }
    std::printf("%d failures\n", g_fail);
    return g_fail;
}
