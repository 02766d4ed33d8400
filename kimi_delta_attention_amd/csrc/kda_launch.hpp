// kda_launch.hpp -- internal launch interface between the C ABI (kda_api.cpp)
// and the kernel translation units.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kda {

struct DecodeParams {
    int N, H, D, W;
    bool x_bf16;
    const void* x;
    const float* conv_w;
    float* conv_state;
    const float* g;
    const float* beta;
    const float* A_log;
    const float* dt_bias;
    float lower_bound;
    int gate_mode;
    int use_qk_l2norm;
    int use_beta_sigmoid;
    float scale;
    float* state;
    float* o;
    const void* out_gate;      // [N, H*D] in x's element type, or nullptr (plain output)
    float out_gate_eps;
    const int32_t* state_slots;  // [N] slot of each sequence in the state pools, or nullptr (slot n)
    int n_slots;                 // pool size when state_slots is given
};

hipError_t launch_decode(const DecodeParams& p, hipStream_t st);

// Full-rank output gate over n_vec head vectors of V values.  Sizes are
// validated by the caller.
struct GateParams {
    int64_t n_vec;             // rows * H
    int V;                     // 32, 64, 128 or 256
    bool o_bf16, g_bf16;       // element types of o / y / dy / dO, and of g / dg
    float eps;
    const void* o;
    const void* g;
    void* y;                   // forward output
    const void* dy;            // reverse mode: upstream gradient and outputs
    void* dO;
    void* dg;
};

hipError_t launch_output_gate(const GateParams& p, hipStream_t st);
// Chains (sequences x heads) from which the chunk forward gates its output in
// the state pass rather than in a pass over o after it.
constexpr int kFusedGateMinChains = 256;
hipError_t launch_output_gate_bwd(const GateParams& p, hipStream_t st);

// Stateful short-conv prefill.  Sizes are validated by the caller.
// Rows of one sequence that one conv-prefill workgroup slides over.
constexpr int kConvBlockRows = 16;

struct ConvParams {
    int B, T, H, D, W;
    int N;                     // number of sequences
    const int32_t* cu_seqlens; // device [N+1] or nullptr (dense)
    bool x_bf16, y_bf16;
    const void* x;             // [rows, 3*H*D]
    const float* conv_w;       // [3*H*D, W]
    float* conv_state;         // [N, 3*H*D, W] in/out, or nullptr
    void* q;                   // [rows, H*D] each
    void* k;
    void* v;
    int block_bound;           // upper bound of the kConvBlockRows-row blocks over all sequences
};

hipError_t launch_conv_prefill(const ConvParams& p, hipStream_t st);

// Chunked path.  Sizes are validated by the caller.
struct ChunkParams {
    int B, T, H, K, V;
    int N;                     // number of sequences
    const int32_t* cu_seqlens; // device [N+1] or nullptr (dense)
    bool bf16;                 // q, k, v, o, dO, dq, dk, dv in bf16 (else fp32)
    const void* q;
    const void* k;
    const void* v;
    const float* g;
    const float* beta;
    const float* A_log;
    const float* dt_bias;
    float scale;
    float lower_bound;         // NaN when absent
    int gate_mode;
    int use_qk_l2norm;
    int use_beta_sigmoid;
    const float* h0;           // [N,H,K,V] or nullptr
    void* o;
    float* ht;                 // [N,H,K,V] or nullptr
    int max_chunks;            // upper bound of chunks per sequence
    int total_chunks_bound;    // upper bound of sum over sequences of chunks
    bool keep;                 // forward writes the backward's slot layout; backward reuses it
    const void* out_gate;      // [rows, H, V] gate input of the fused output gate, or nullptr
    bool out_gate_bf16;        // its element type (bf16, else fp32)
    float out_gate_eps;
};

struct ChunkGrads {
    const void* dO;
    const float* dht;          // [N,H,K,V] or nullptr
    void* dq;
    void* dk;
    void* dv;
    float* dg;
    float* dbeta;
    float* dh0;                // or nullptr
    float* dA_log;             // or nullptr
    float* ddt_bias;           // or nullptr
};

size_t chunk_fwd_workspace(const ChunkParams& p);  // of the forward's own layout

// Bytes of the library's own device scratch (kda_noalloc.hip), one array per
// GPU; kda.h states the same value as KDA_NOALLOC_SCRATCH_BYTES.
constexpr size_t kNoAllocScratchBytes = static_cast<size_t>(192) << 20;
// Device address of the current device's scratch array (looked up once per
// device, thread-safe).
hipError_t noalloc_workspace(void** ptr);
// stage < 0 runs every stage; 0 = prep, 1 = state pass.  With p.keep the
// forward writes the backward's layout (chunk_bwd_workspace bytes).
hipError_t launch_chunk_fwd(const ChunkParams& p, void* ws, hipStream_t st, int stage = -1);

size_t chunk_bwd_workspace(const ChunkParams& p);
// stage < 0 runs every stage; 0 prep, 1 state pass (stores states), 2 reverse
// state pass, 3 V-local gradients, 4 K-local gradients.  With p.keep stages 0
// and 1 were done by the forward and launch nothing.
constexpr int kBwdStages = 5;
hipError_t launch_chunk_bwd(const ChunkParams& p, const ChunkGrads& gr, void* ws, hipStream_t st, int stage = -1);

}  // namespace kda
