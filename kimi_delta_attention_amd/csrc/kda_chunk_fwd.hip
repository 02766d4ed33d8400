// kda_chunk_fwd.hip -- chunkwise-parallel KDA forward on gfx950: the
// launch sequence of the prep and state kernels (kda_chunk_kernels.hpp).
#include "kda_chunk_kernels.hpp"

namespace kda {

// ------------------------------------------------------------------ host side
template <int K, bool BF, int V = K>
static size_t prep_bytes(const ChunkParams& p) {
    return static_cast<size_t>(p.total_chunks_bound) * p.H * PrepLayout<K, BF, V>::kBytes;
}

size_t chunk_fwd_workspace(const ChunkParams& p) {
    size_t prep = 0;
    if (p.K == 32 && p.V == 64)
        return chunk_off_bytes(p) + (p.bf16 ? prep_bytes<32, true, 64>(p) : prep_bytes<32, false, 64>(p));
    if (p.K != p.V) return 0;
    switch (p.K) {
        case 32: prep = p.bf16 ? prep_bytes<32, true>(p) : prep_bytes<32, false>(p); break;
        case 64: prep = p.bf16 ? prep_bytes<64, true>(p) : prep_bytes<64, false>(p); break;
        case 128: prep = p.bf16 ? prep_bytes<128, true>(p) : 0; break;
        default: return 0;
    }
    return chunk_off_bytes(p) + prep;
}

// KEEP writes the backward's slot layout (BwdExtra): the prep also stores
// KE, T and AK, and the state pass also stores every chunk's entry state, so
// that the backward can skip its stages 0 and 1.
template <int K, int V, int BV, bool BF, bool KEEP>
static hipError_t run_fwd(const ChunkParams& p, void* ws, hipStream_t st, int stage) {
    uint8_t* w8 = static_cast<uint8_t*>(ws);
    int32_t* chunk_off = reinterpret_cast<int32_t*>(w8);
    uint8_t* prep = w8 + chunk_off_bytes(p);
    const int64_t sb = static_cast<int64_t>(KEEP ? BwdExtra<K, BF, V>::kBytes : PrepLayout<K, BF, V>::kBytes);
    if (stage < 0 || stage == 0) {
        if (p.cu_seqlens)
            hipLaunchKernelGGL(plan_chunks_kernel, dim3(1), dim3(kPlanThreads), 0, st, p.cu_seqlens, p.N, p.T, chunk_off,
                               p.total_chunks_bound);
        const int64_t nblk = static_cast<int64_t>(p.total_chunks_bound) * p.H;
        if (nblk > 0)
            hipLaunchKernelGGL((chunk_prep_kernel<K, BF, KEEP, V>), dim3(prep_grid<K, BF, KEEP, V>(nblk)),
                               dim3(prep_threads(K)), 0, st, p, chunk_off, prep, sb, nblk);
    }
    // The output gate needs a head's whole row of V outputs.  With enough
    // chains to fill the chip, the state pass takes one workgroup per head and
    // gates each row before its store; with fewer, the plain pass (V split
    // over workgroups) writes o and the gate runs over it in place right after:
    // measured equal at 256 chains and faster below (e.g. 64 chains of the
    // packed 8192-token batch: 192 against 308 us).
    const bool gate_in_state = p.out_gate && p.N * p.H >= kFusedGateMinChains;
    if ((stage < 0 || stage == 1) && gate_in_state) {
        if constexpr (!KEEP) {
            const int chains = p.N * p.H;
            if constexpr (K == 128 && V == 128 && BF) {
                if (p.out_gate_bf16)
                    hipLaunchKernelGGL((chunk_state_fwd_gate_kernel<true>), dim3(chains), dim3(kGateStateThreads), 0,
                                       st, p, chunk_off, prep, sb);
                else
                    hipLaunchKernelGGL((chunk_state_fwd_gate_kernel<false>), dim3(chains), dim3(kGateStateThreads), 0,
                                       st, p, chunk_off, prep, sb);
            } else {
                hipLaunchKernelGGL((chunk_state_fwd_kernel<K, V, V, BF, false, true, kThreads, true>),
                                   dim3(chain_grid(chains, 1)), dim3(kThreads), 0, st, p, chunk_off, prep, sb);
            }
        }
        return hipGetLastError();
    }
    if (stage < 0 || stage == 1) {
        // few chains (no more workgroups than CUs): 8 waves per chain shorten
        // each chunk step; otherwise 4 waves let two chains share a CU
        const int grid = chain_grid(p.N * p.H, V / BV);
        if constexpr (K == 128 && V == 128 && BF) {
            if (state_pc_bv(p.N * p.H) == 32) {
                if (grid > 0)
                    hipLaunchKernelGGL((chunk_state_fwd_pc_kernel<KEEP, true, 32>), dim3(grid),
                                       dim3(state_pc_threads(32)), 0, st, p, chunk_off, prep, sb);
            } else {
                hipLaunchKernelGGL((chunk_state_fwd_pc_kernel<KEEP, true, 64>), dim3(chain_grid(p.N * p.H, 2)),
                                   dim3(state_pc_threads(64)), 0, st, p, chunk_off, prep, sb);
            }
        } else if (grid > 0 && grid <= kPersistentGrid)
            hipLaunchKernelGGL((chunk_state_fwd_kernel<K, V, BV, BF, KEEP, true, 512>), dim3(grid), dim3(512), 0,
                               st, p, chunk_off, prep, sb);
        else if (grid > 0)
            hipLaunchKernelGGL((chunk_state_fwd_kernel<K, V, BV, BF, KEEP, true>), dim3(grid), dim3(kThreads), 0,
                               st, p, chunk_off, prep, sb);
        if (p.out_gate && !KEEP) {  // the gate over o, in place
            GateParams gp{};
            gp.n_vec = static_cast<int64_t>(p.cu_seqlens ? p.T : static_cast<int64_t>(p.B) * p.T) * p.H;
            gp.V = V;
            gp.o_bf16 = BF;
            gp.g_bf16 = p.out_gate_bf16;
            gp.eps = p.out_gate_eps;
            gp.o = p.o;
            gp.g = p.out_gate;
            gp.y = p.o;
            const hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
            return launch_output_gate(gp, st);
        }
    }
    return hipGetLastError();
}

template <int K, int V, int BV, bool BF>
static hipError_t run_fwd_any(const ChunkParams& p, void* ws, hipStream_t st, int stage) {
    return p.keep ? run_fwd<K, V, BV, BF, true>(p, ws, st, stage) : run_fwd<K, V, BV, BF, false>(p, ws, st, stage);
}

hipError_t launch_chunk_fwd(const ChunkParams& p, void* ws, hipStream_t st, int stage) {
    if (p.K == 32 && p.V == 64)
        return p.bf16 ? run_fwd_any<32, 64, 16, true>(p, ws, st, stage) : run_fwd_any<32, 64, 16, false>(p, ws, st, stage);
    if (p.K != p.V) return hipErrorInvalidValue;
    switch (p.K) {
        case 32:
            return p.bf16 ? run_fwd_any<32, 32, 16, true>(p, ws, st, stage) : run_fwd_any<32, 32, 16, false>(p, ws, st, stage);
        case 64:
            return p.bf16 ? run_fwd_any<64, 64, 32, true>(p, ws, st, stage) : run_fwd_any<64, 64, 32, false>(p, ws, st, stage);
        case 128: return p.bf16 ? run_fwd_any<128, 128, 32, true>(p, ws, st, stage) : hipErrorInvalidValue;
        default: return hipErrorInvalidValue;
    }
}

}  // namespace kda
