// kda_chunk_bwd.hip -- chunked KDA backward on gfx950.
//
// The pages give no backward; this is the adjoint of the chunk form in
// kda_chunk_kernels.hpp, written per chunk with QE = scale q^ e^G,
// KE = k^ e^G, KD = k^ e^(G_last - G), TB = T diag(beta), MS = scale M,
// gam = e^G_last and, for the entry state S and the exit-state gradient dS':
//   Y  = v - KE S            D  = TB Y
//   O  = QE S + MS D         S' = gam * S + KD^T D
// which gives (all products column-local in V except where summed over V)
//   dD  = KD dS' + MS^T dO            dY = TB^T dD            dv = dY
//   dS  = gam * dS' + QE^T dO - KE^T dY = gam * dS' + QE^T dO - W^T dD
//                                        (reverse pass; W = TB KE from the prep)
//   dQE = dO S^T   dKE = -dY S^T   dKD = D dS'^T   dMS = dO D^T   dTB = dD Y^T
//   dgam = rowsum(dS' * S)
// then, through the prologue of the chunk,
//   dT = dTB diag(beta), dbeta_j += sum_i dTB_ij T_ij
//   dA = -T^T dT T^T (strictly lower), dbeta_i += sum_j dA_ij Ak_ij, dAk = diag(beta) dA
//   score rule for X_ij = sum_c x_ic k_jc e^(G_ic - G_jc) with gradient dX:
//     dx_i += sum_j dX_ij k_j e^(G_i - G_j),  dk_j += sum_i dX_ij x_i e^(G_i - G_j),
//     dG_i += x_i * (first sum),  dG_j -= k_j * (second sum)
//   (x = q^ for M, x = k^ for Ak), the element-wise terms of QE, KE, KD, gam,
//   the reverse cumulative sum of dG inside the chunk, and the chain rule of
//   the gate, the beta sigmoid and the L2 norm.
//
// Kernels, in launch order (stage numbers of kda_chunk_bwd_stage):
//   0 prep       the forward's prep kernel, also writing T and Ak;
//   1 fstate     the forward state pass, storing every chunk's entry state;
//   2 bstate     the reverse state pass, storing every chunk's exit-state
//                gradient (sequential over chunks, parallel over sequence x
//                head x V-column block), writing d(initial state);
//   3 vlocal     per (chunk, head): dv and the V-summed operand gradients;
//   4 klocal     per (chunk, head): dq, dk, dg, dbeta (and the gate-parameter
//                shares), plus the reduction of d(A_log), d(dt_bias).
// The score rule runs on MFMA products with the per-sub-block factorisation of
// the forward: sub-block pairs through the row before the later block, diagonal
// sub-blocks through the row before them when their decay span allows, else by
// the level decomposition (every factor at most 1), so any gate is exact.  The
// fp32 kernel forms the score rule pairwise instead.
#include "kda_chunk_kernels.hpp"

namespace kda {

// ------------------------------------------------------------------ reverse state pass
// Per chunk in reverse, with dS' the gradient of the state leaving the chunk:
//   dD = KD dS' + MS^T dO,   dS = GC * dS' + QE^T dO - W^T dD
// (W^T dD = (k exp(G))^T TB^T dD).  dS' is stored in the chunk's slot.
template <int K, int V, int BV, bool BF>
__global__ __launch_bounds__(kThreads) void chunk_state_bwd_kernel(ChunkParams p, ChunkGrads gr,
                                                                   const int32_t* chunk_off, uint8_t* ws,
                                                                   int64_t slot_bytes) {
    using MM = Mma<BF>;
    using ET = typename MM::ET;
    using IT = typename std::conditional<BF, uint16_t, float>::type;
    using L = PrepLayout<K, BF, V>;
    using X = BwdExtra<K, BF, V>;
    constexpr int LDK = K + MM::PAD;
    constexpr int LDC = kChunk + MM::PAD;
    constexpr int NCT = BV / 16;
    constexpr int NST = (K / 16) * NCT;
    constexpr int SPW = (NST + 3) / 4;
    constexpr int NVB = V / BV;

    __shared__ __attribute__((aligned(16))) ET QEt[K][LDC];       // QE^T: A of QE^T dO
    __shared__ __attribute__((aligned(16))) ET Wt[K][LDC];        // W^T:  A of W^T dD
    __shared__ __attribute__((aligned(16))) ET KDn[kChunk][LDK];  // A of KD dS'
    __shared__ __attribute__((aligned(16))) ET MSt[kChunk][LDC];  // MS^T: A of MS^T dO
    __shared__ __attribute__((aligned(16))) ET dSt[BV][LDK];      // dS'^T: B of KD dS'
    __shared__ __attribute__((aligned(16))) ET dOt[BV][LDC];
    __shared__ __attribute__((aligned(16))) ET dDt[BV][LDC];
    __shared__ __attribute__((aligned(16))) float gC[K];

    int chain, vb;
    if (!chain_of_block(blockIdx.x, p.N * p.H, NVB, chain, vb)) return;
    const int H = p.H;
    const int n = chain / H, h = chain % H;
    int64_t start;
    int len;
    seq_bounds(p, n, start, len);
    const int nc = chain_chunks(p, chunk_off, n, len);
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    const int v0 = vb * BV;
    const int64_t sbase = (static_cast<int64_t>(n) * H + h) * K * V;
    const int64_t slot0 = chunk_slot(p, chunk_off, n, 0);

    Seg<ET, kChunk, K, true> sQE, sW;
    Seg<ET, kChunk, K, false> sKD;
    Seg<ET, kChunk, kChunk, true> sMS;
    Seg<ET, kChunk, BV, true> sdO;
    Seg<float, 1, K, false> sGC;
    const ET* dOg = static_cast<const ET*>(gr.dO);
    auto prefetch = [&](int jc) {
        const uint8_t* base = ws + ((slot0 + jc) * H + h) * slot_bytes;
        sQE.load(reinterpret_cast<const ET*>(base + L::kQE), K, t);
        sW.load(reinterpret_cast<const ET*>(base + L::kW), K, t);
        sKD.load(reinterpret_cast<const ET*>(base + L::kKD), K, t);
        sMS.load(reinterpret_cast<const ET*>(base + L::kMS), kChunk, t);
        sGC.load(reinterpret_cast<const float*>(base + L::kGC), K, t);
        sdO.load(dOg + ((start + static_cast<int64_t>(jc) * kChunk) * H + h) * V + v0,
                 static_cast<int64_t>(H) * V, t, min(kChunk, len - jc * kChunk));
    };

    f32x4 dS[SPW];
#pragma unroll
    for (int m = 0; m < SPW; ++m) {
        const int tt = w + 4 * m;
        const int rt = tt / NCT, ct = tt % NCT;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            float v = 0.f;
            if (tt < NST && gr.dht) v = gr.dht[sbase + (16 * rt + 4 * (lane >> 4) + r) * V + v0 + 16 * ct + (lane & 15)];
            dS[m][r] = v;
        }
    }
    if (nc > 0) prefetch(nc - 1);
    const int klo = (16 * w / MM::KS) * MM::KS;
    for (int jc = nc - 1; jc >= 0; --jc) {
        sQE.store(&QEt[0][0], LDC, t);
        sW.store(&Wt[0][0], LDC, t);
        sKD.store(&KDn[0][0], LDK, t);
        sMS.store(&MSt[0][0], LDC, t);
        sGC.store(&gC[0], K, t);
        sdO.store(&dOt[0][0], LDC, t);
        uint8_t* base = ws + ((slot0 + jc) * H + h) * slot_bytes;
        ET* gDS = reinterpret_cast<ET*>(base + X::kDS);
#pragma unroll
        for (int m = 0; m < SPW; ++m) {
            const int tt = w + 4 * m;
            if (tt < NST) {
                const int rt = tt / NCT, ct = tt % NCT;
                tile_store_t<MM>(gDS + v0 * K, K, 16 * rt, 16 * ct, dS[m], lane);  // dS'^T rows
                tile_store_t<MM>(&dSt[0][0], LDK, 16 * rt, 16 * ct, dS[m], lane);
            }
        }
        __syncthreads();
        if (jc > 0) prefetch(jc - 1);

        // dD = KD dS' + MS^T dO   (rows 16w..; MS^T is upper triangular: k >= 16w)
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            acc = gemm<MM>(&KDn[0][0], LDK, 16 * w, &dSt[0][0], LDK, 16 * ct, 0, K, acc, lane);
            acc = gemm<MM>(&MSt[0][0], LDC, 16 * w, &dOt[0][0], LDC, 16 * ct, klo, kChunk, acc, lane);
            tile_store_t<MM>(&dDt[0][0], LDC, 16 * w, 16 * ct, acc, lane);
        }
        __syncthreads();

        // dS = GC * dS' + QE^T dO - W^T dD
#pragma unroll
        for (int m = 0; m < SPW; ++m) {
            const int tt = w + 4 * m;
            if (tt < NST) {
                const int rt = tt / NCT, ct = tt % NCT;
                f32x4 neg = {0.f, 0.f, 0.f, 0.f};
                neg = gemm<MM>(&Wt[0][0], LDC, 16 * rt, &dDt[0][0], LDC, 16 * ct, 0, kChunk, neg, lane);
#pragma unroll
                for (int r = 0; r < 4; ++r) dS[m][r] = dS[m][r] * gC[16 * rt + 4 * (lane >> 4) + r] - neg[r];
                dS[m] = gemm<MM>(&QEt[0][0], LDC, 16 * rt, &dOt[0][0], LDC, 16 * ct, 0, kChunk, dS[m], lane);
            }
        }
        __syncthreads();
    }
    if (gr.dh0) {
#pragma unroll
        for (int m = 0; m < SPW; ++m) {
            const int tt = w + 4 * m;
            if (tt < NST) {
                const int rt = tt / NCT, ct = tt % NCT;
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    gr.dh0[sbase + (16 * rt + 4 * (lane >> 4) + r) * V + v0 + 16 * ct + (lane & 15)] = dS[m][r];
            }
        }
    }
}

// Reverse state pass for K = V = 128 in bf16, BV (32 or 64) value columns per
// workgroup, state_pc_threads(BV) threads: the producer/consumer form of
// chunk_state_fwd_pc_kernel.  Waves 0 .. BV/16 - 1 (consumers) each own a
// 16-column strip of dS' over all 128 rows.  dD = KD dS' + MS^T dO takes dS'
// from registers as its B operand.  The token-row products QE^T dO and W^T dD
// take dO, read transposed, and -dD, formed in registers, as B.  The last two
// waves (producers) copy each chunk's operand tiles and dO block into LDS a
// chunk ahead, warm L2 a few chunks ahead, and at BV = 32 store the staged dS'
// of the chunk before; at BV = 64 (the block count of state_pc_bv) the
// consumers store their dS' strips themselves, since the staging would not
// fit the LDS beside the operand buffers.
template <int BV>
struct StatePcBwd {
    static constexpr int oW = 0, oQE = 16384, oKD = 32768, oMS = 49152, oDO = 57344, oGC = oDO + 128 * BV;
    static constexpr int kBuf = oGC + 512;  // one chunk's operand tiles and dO block
};

template <int BV>
__global__ __launch_bounds__(state_pc_threads(BV)) void chunk_state_bwd_pc_kernel(ChunkParams p, ChunkGrads gr,
                                                                                  const int32_t* chunk_off,
                                                                                  uint8_t* ws, int64_t slot_bytes) {
    static_assert(BV == 32 || BV == 64, "32- or 64-column blocks");
    using Z = StatePcBwd<BV>;
    using L = PrepLayout<128, true>;
    using X = BwdExtra<128, true>;
    constexpr int K = 128, V = 128, NVB = V / BV, NCW = BV / 16;
    constexpr bool STAGE = BV == 32;  // dS' staged for the producers
    constexpr int WA = BV == 32 ? kWarmAhead : kWarmAhead64;
    // L2 warm-up lines of a chunk: QE, W, KD (contiguous), MS, GC, then the
    // dO rows (two lines per head row), split over the chain's NVB workgroups
    constexpr int NL = 384 + 64 + 4 + 128;
    constexpr int NWARM = (NL + NVB * 128 - 1) / (NVB * 128);
    __shared__ __attribute__((aligned(1024))) uint8_t smb[2 * Z::kBuf];
    __shared__ __attribute__((aligned(1024))) uint8_t sms[STAGE ? 2 * 8192 : 16];  // dS'^T staging [32][128] per parity
    __shared__ __attribute__((aligned(256))) uint8_t smj[256];

    int chain, vb;
    if (!chain_of_block(blockIdx.x, p.N * p.H, NVB, chain, vb)) return;
    const int H = p.H;
    const int n = chain / H, h = chain % H;
    int64_t start;
    int len;
    seq_bounds(p, n, start, len);
    const int nc = chain_chunks(p, chunk_off, n, len);
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int lg = lane >> 4, m = lane & 15;
    const int v0 = vb * BV;
    const int64_t slot0 = chunk_slot(p, chunk_off, n, 0);
    const int64_t sbase = (static_cast<int64_t>(n) * H + h) * K * V;
    const bool prod = w >= NCW;
    const int pw = w - NCW;
    const uint16_t* dOg = static_cast<const uint16_t*>(gr.dO);
    auto slot = [&](int jc) { return ws + ((slot0 + jc) * H + h) * slot_bytes; };
    auto rows_in = [&](int jc) { return min(kChunk, len - jc * kChunk); };  // >= 1 for jc < nc

    // ---- producer: chunk jc's operand tiles and dO block into buffer jc & 1
    auto fetch = [&](int jc) {
        const uint8_t* base = slot(jc);
        uint8_t* buf = smb + (jc & 1) * Z::kBuf;
#pragma unroll
        for (int qq = 0; qq < 8; ++qq) {
            const int q = 2 * qq + pw;
            dma_tile_piece<128>(reinterpret_cast<const uint16_t*>(base + L::kKD), K, buf + Z::oKD, q, lane);
            dma_tile_piece<128>(reinterpret_cast<const uint16_t*>(base + L::kQE), K, buf + Z::oQE, q, lane);
            dma_tile_piece<128>(reinterpret_cast<const uint16_t*>(base + L::kW), K, buf + Z::oW, q, lane);
        }
#pragma unroll
        for (int qq = 0; qq < 4; ++qq)
            dma_tile_piece<64>(reinterpret_cast<const uint16_t*>(base + L::kMS), kChunk, buf + Z::oMS, 2 * qq + pw,
                                lane);
        const uint16_t* dO0 = dOg + ((start + static_cast<int64_t>(jc) * kChunk) * H + h) * V + v0;
#pragma unroll
        for (int qq = 0; qq < BV / 16; ++qq)
            dma_tile_piece<BV>(dO0, static_cast<int64_t>(H) * V, buf + Z::oDO, 2 * qq + pw, lane, rows_in(jc));
        if (pw == 1 && lane < 32) dma16(base + L::kGC + 16 * lane, buf + Z::oGC);
    };
    // ---- producer: chunk jc's dS' from staging jc & 1, as whole transposed
    // rows (column v of dS': 128 values, 256 bytes)
    auto drain = [&](int jc) {
        const uint8_t* st = sms + (jc & 1) * 8192;
        bf16x8 xs[4];
#pragma unroll
        for (int q = 0; q < 4; ++q)  // rows 16 pw + 4 q + lane / 16, 16-byte chunk lane % 16
            xs[q] = *reinterpret_cast<const bf16x8*>(st + swz_off<128>(16 * pw + 4 * q + lg, 8 * m));
        uint16_t* gD = reinterpret_cast<uint16_t*>(slot(jc) + X::kDS) + v0 * K;
#pragma unroll
        for (int q = 0; q < 4; ++q) *reinterpret_cast<bf16x8*>(gD + (16 * pw + 4 * q + lg) * K + 8 * m) = xs[q];
    };
    // ---- producer: one 4-byte copy per 128-byte line of chunk jc's inputs
    auto warm = [&](int jc) {
        const uint8_t* base = slot(jc);
        const int rv = rows_in(jc);
#pragma unroll
        for (int i = 0; i < NWARM; ++i) {
            int l = NVB * ((2 * i + pw) * 64 + lane) + vb;
            l = l < NL ? l : NL - 1;
            const void* a;
            if (l < 384) a = base + L::kQE + 128 * l;
            else if (l < 448) a = base + L::kMS + 128 * (l - 384);
            else if (l < 452) a = base + L::kGC + 128 * (l - 448);
            else {
                const int r = min((l - 452) >> 1, rv - 1);
                a = dOg + ((start + static_cast<int64_t>(jc) * kChunk + r) * H + h) * V + 64 * ((l - 452) & 1);
            }
            __builtin_amdgcn_global_load_lds(a, (lds_void_t*)smj, 4, 0, 0);
        }
    };

    // ---- consumer: dS' strip, tile t = rows 16 t + 4 lg + r, column 16 w + m
    f32x4 dS[8];
    int offA[4];      // [64][128] row fragment, k-step s, row tile 0 (+4096 per row tile)
    int offT[8][2];   // [64][128] transposed fragment halves, column tile t, k-step 0 (+8192 per k-step)
    int offMT[4][2];  // [64][64] transposed fragment halves, column tile j, k-step 0 (+4096 per k-step)
    int offD[2];      // [64][BV] dO, transposed halves, k-step 0 (+64 BV per k-step)
#pragma unroll
    for (int s = 0; s < 4; ++s) offA[s] = swz_off<128>(m, 32 * s + 8 * lg);
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
        const int r = 8 * lg + 4 * hh + (m >> 2);
#pragma unroll
        for (int t = 0; t < 8; ++t) offT[t][hh] = swz_off<128>(r, 16 * t + 4 * (m & 3));
#pragma unroll
        for (int j = 0; j < 4; ++j) offMT[j][hh] = swz_off<64>(r, 16 * j + 4 * (m & 3));
        offD[hh] = swz_off<BV>(r, 16 * w + 4 * (m & 3));
    }
    auto rdA = [](const uint8_t* tile, int off) { return *reinterpret_cast<const bf16x8*>(tile + off); };
    auto rdT = [](const uint8_t* tile, int off0, int off1) {
        const bf16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(tile + off0));
        const bf16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(tile + off1));
        return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    };
    auto step = [&](int jc) {
        const uint8_t* buf = smb + (jc & 1) * Z::kBuf;
        uint8_t* st = sms + (jc & 1) * 8192;
        bf16x8 Sb[4];  // dS' as the B operand over state rows; also stored (lane group lg: k = 32 s + 8 lg ..)
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            Sb[s] = frag_acc_nat(dS[2 * s], dS[2 * s + 1]);
            if (STAGE) *reinterpret_cast<bf16x8*>(st + swz_off<128>(16 * w + m, 32 * s + 8 * lg)) = Sb[s];
        }
        if (!STAGE) {  // straight to the slot's transposed dS'
            uint16_t* gD = reinterpret_cast<uint16_t*>(slot(jc) + X::kDS) + (v0 + 16 * w + m) * K;
#pragma unroll
            for (int s = 0; s < 4; ++s) *reinterpret_cast<bf16x8*>(gD + 32 * s + 8 * lg) = Sb[s];
        }
        // The LDS reads are issued in batches ahead of the products that use
        // them (scheduling barriers keep that order).
        // dO block as the B operand over token rows (zero past the sequence
        // end), the MS^T fragments, the decay factors and the first KD fragments
        bf16x8 dOb[2];
#pragma unroll
        for (int s = 0; s < 2; ++s) dOb[s] = rdT(buf + Z::oDO + 64 * BV * s, offD[0], offD[1]);
        bf16x8 fm[6];
#pragma unroll
        for (int jt = 0, q = 0; jt < 4; ++jt)
#pragma unroll
            for (int s = jt >> 1; s < 2; ++s, ++q) fm[q] = rdT(buf + Z::oMS + 4096 * s, offMT[jt][0], offMT[jt][1]);
        f32x4 g[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) g[t] = *reinterpret_cast<const f32x4*>(buf + Z::oGC + 4 * (16 * t + 4 * lg));
        bf16x8 fa[2][4];
        auto load_a = [&](int s, bf16x8* f) {
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) f[rt] = rdA(buf + Z::oKD + 4096 * rt, offA[s]);
        };
        load_a(0, fa[0]);
        __builtin_amdgcn_sched_barrier(0);
        const int rv = rows_in(jc);
        if (rv < kChunk) {
#pragma unroll
            for (int s = 0; s < 2; ++s)
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    if (32 * s + 8 * lg + j >= rv) dOb[s][j] = static_cast<__bf16>(0.f);
        }
        // dD = KD dS' + MS^T dO   (MS^T upper triangular), KD one k-step ahead
        f32x4 dd[4];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) dd[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            if (s < 3) load_a(s + 1, fa[(s + 1) & 1]);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int rt = 0; rt < 4; ++rt)
                dd[rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[s & 1][rt], Sb[s], dd[rt], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
        // QE^T and W^T fragments of one state-row tile: [QE s0, QE s1, W s0, W s1]
        bf16x8 fq[2][4];
        auto load_q = [&](int t, bf16x8* f) {
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                f[s] = rdT(buf + Z::oQE + 8192 * s, offT[t][0], offT[t][1]);
                f[2 + s] = rdT(buf + Z::oW + 8192 * s, offT[t][0], offT[t][1]);
            }
        };
        load_q(0, fq[0]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int jt = 0, q = 0; jt < 4; ++jt)
#pragma unroll
            for (int s = jt >> 1; s < 2; ++s, ++q)
                dd[jt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fm[q], dOb[s], dd[jt], 0, 0, 0);
        const bf16x8 nDb[2] = {frag_acc_nat(-dd[0], -dd[1]), frag_acc_nat(-dd[2], -dd[3])};
        // dS = GC dS' + QE^T dO - W^T dD, one state-row tile of fragments ahead
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            if (t < 7) load_q(t + 1, fq[(t + 1) & 1]);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int r = 0; r < 4; ++r) dS[t][r] *= g[t][r];
#pragma unroll
            for (int s = 0; s < 2; ++s)
                dS[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fq[t & 1][s], dOb[s], dS[t], 0, 0, 0);
#pragma unroll
            for (int s = 0; s < 2; ++s)
                dS[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fq[t & 1][2 + s], nDb[s], dS[t], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    if (prod) {
        if (nc > 0) fetch(nc - 1);
        wait_vmem_all();
    } else {
#pragma unroll
        for (int t = 0; t < 8; ++t) dS[t] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (gr.dht) {
#pragma unroll
            for (int t = 0; t < 8; ++t)
#pragma unroll
                for (int r = 0; r < 4; ++r) dS[t][r] = gr.dht[sbase + (16 * t + 4 * lg + r) * V + v0 + 16 * w + m];
        }
    }
    __syncthreads();
    // One loop per role (each wave passes the same nc barriers): a shared loop
    // body makes the compiler keep both roles' values live at once.
    if (prod) {
        for (int jc = nc - 1; jc >= 0; --jc) {
            // staging reads before this step's copies (the compiler would wait
            // for the copies before later LDS reads); the warm-up loads are
            // issued last and are the only ones allowed to stay in flight
            if (STAGE && jc + 1 < nc) drain(jc + 1);
            if (jc > 0) fetch(jc - 1);
            __builtin_amdgcn_sched_barrier(0);
            warm(jc >= WA ? jc - WA : jc);
            __builtin_amdgcn_sched_barrier(0);
            wait_vmem<NWARM>();
            barrier_lds();
        }
    } else {
        for (int jc = nc - 1; jc >= 0; --jc) {
            step(jc);
            barrier_lds();
        }
    }
    if (prod) {
        if (STAGE && nc > 0) drain(0);
    } else if (gr.dh0) {
#pragma unroll
        for (int t = 0; t < 8; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) gr.dh0[sbase + (16 * t + 4 * lg + r) * V + v0 + 16 * w + m] = dS[t][r];
    }
}

// ------------------------------------------------------------------ V-local gradients
// Threads of a V-local workgroup (its LDS allows one per CU): the bf16
// variant takes 8 waves, two per 16-row tile splitting the column tiles, so
// that one wave's LDS and memory chains overlap another's products.
__host__ __device__ constexpr int vlocal_threads(bool bf) { return bf ? 512 : 256; }

// Per V-column block of BV columns: Y = v - KE S, dD = KD dS' + MS^T dO,
// D = TB Y, dY = TB^T dD (= dv), and the V-summed products dQE, dKE, dKD,
// dMS, dTB, dgam accumulate over the blocks.  The next block's S, dS', dO and
// v are requested before the current block's products.  dgam (per key, the
// sum over the value columns of S dS') is formed from the blocks' S and dS'
// vectors while they are in registers: each thread keeps the partial sums of
// its vector's keys, and the BV threads that hold one key vector's columns
// add theirs at the end of the item, within their wave.  Every operand stays
// in LDS in the layout it arrives in: products that need a transposed operand
// (MS^T, TB^T, and S, dS', dO, Y, dD as [k][n] B operands) read it through
// the transposing LDS read (load_kn).
//
// Persistent over the (slot, head) items like the prep kernel: the next
// item's KE, KD, TB and MS are requested once the current ones are in LDS,
// and its first block's S, dS', dO and v during the current item's last
// block.
// One persistent workgroup per CU: at K = 128 the LDS allows no second one,
// and at smaller K the registers of the item loop do not.
__host__ inline unsigned vlocal_grid(int64_t n_items) {
    return static_cast<unsigned>(n_items < kPersistentGrid ? n_items : kPersistentGrid);
}

template <int K, int V, int BV, bool BF>
__global__ __launch_bounds__(vlocal_threads(BF)) void chunk_bwd_vlocal_kernel(ChunkParams p, ChunkGrads gr,
                                                                              const int32_t* chunk_off,
                                                                              uint8_t* ws, int64_t slot_bytes,
                                                                              int64_t n_items) {
    using MM = Mma<BF>;
    using ET = typename MM::ET;
    using IT = typename std::conditional<BF, uint16_t, float>::type;
    using L = PrepLayout<K, BF, V>;
    using X = BwdExtra<K, BF, V>;
    constexpr int NT = vlocal_threads(BF);
    constexpr int WPR = NT / 256;  // waves per 16-row tile
    constexpr int LDK = K + MM::PAD;
    constexpr int LDC = kChunk + MM::PAD;
    constexpr int LDB = BV + MM::PAD;
    constexpr int NCT = BV / 16;   // column tiles of a [64][BV] block
    constexpr int NKT = K / 16;    // column tiles of a [64][K] product
    constexpr int VE = 16 / sizeof(ET);          // elements per 16-byte vector
    constexpr int VPR = BV / VE;                 // vectors per block row
    constexpr int NVS = K * VPR;                 // vectors of an S (or dS') block (rows of S^T, K long)
    constexpr int NVO = kChunk * VPR;            // vectors of a dO block
    constexpr int PS = (NVS + NT - 1) / NT;
    constexpr int PO = (NVO + NT - 1) / NT;
    constexpr int TW = (NCT + WPR - 1) / WPR;    // column tiles per wave in a block
    constexpr int AW = NKT / WPR;                // [64][K] accumulator tiles per wave
    constexpr int CW = 4 / WPR;                  // [64][64] accumulator tiles per wave
    static_assert(BV % MM::KS == 0, "products contract over the V block: it must hold whole MFMA k-steps");
    static_assert(BV % VE == 0 && NKT % WPR == 0, "block shapes");

    __shared__ __attribute__((aligned(16))) ET KEn[kChunk][LDK];
    __shared__ __attribute__((aligned(16))) ET KDn[kChunk][LDK];
    __shared__ __attribute__((aligned(16))) ET TBn[kChunk][LDC];
    __shared__ __attribute__((aligned(16))) ET MSn[kChunk][LDC];
    __shared__ __attribute__((aligned(16))) ET St[BV][LDK];   // S^T block: row = value column, K keys
    __shared__ __attribute__((aligned(16))) ET dSt[BV][LDK];
    __shared__ __attribute__((aligned(16))) ET dOn[kChunk][LDB];
    __shared__ __attribute__((aligned(16))) ET Yn[kChunk][LDB];
    __shared__ __attribute__((aligned(16))) ET Dn[kChunk][LDB];
    __shared__ __attribute__((aligned(16))) ET dDn[kChunk][LDB];
    __shared__ __attribute__((aligned(16))) ET dYn[kChunk][LDB];

    const int H = p.H;
    const int64_t GS = gridDim.x;
    const IT* dOg = static_cast<const IT*>(gr.dO);
    const IT* vg = static_cast<const IT*>(p.v);
    IT* dvg = static_cast<IT*>(gr.dv);

    // where an item is
    struct Loc {
        bool ok;
        int h, rows;
        int64_t rbase;  // global row of the chunk's first row
        uint8_t* base;  // the item's workspace slot
    };
    auto map_entry = [&](int64_t item) -> int4 {
        int4 e = {-1, 0, 0, 0};
        if (p.cu_seqlens && item < n_items)
            e = reinterpret_cast<const int4*>(reinterpret_cast<const uint8_t*>(chunk_off) + plan_map_offset(p.N))[item / H];
        return e;
    };
    auto decode = [&](int64_t item, int4 e) -> Loc {
        Loc l{false, 0, 0, 0, ws};
        if (item >= n_items) return l;
        int n, j, len;
        int64_t start;
        const int slot = static_cast<int>(item / H);
        if (p.cu_seqlens) {
            n = e.x;
            j = e.y;
            start = e.z;
            len = e.w;
            if (n < 0) return l;
        } else {
            const int nc = n_chunks(p.T);
            n = slot / nc;
            j = slot % nc;
            start = static_cast<int64_t>(n) * p.T;
            len = p.T;
            if (n >= p.N) return l;
        }
        l.ok = true;
        l.h = item_head(item, H, GS, p.gate_mode != GATE_LOGDECAY);
        l.rows = min(kChunk, len - j * kChunk);
        l.rbase = start + static_cast<int64_t>(j) * kChunk;
        l.base = ws + (static_cast<int64_t>(slot) * H + l.h) * slot_bytes;
        return l;
    };

    // an item's KE, KD, TB and MS in registers on their way to LDS
    Seg<ET, kChunk, K, false, NT> cKE, cKD;
    Seg<ET, kChunk, kChunk, false, NT> cTB, cMS;
    auto fetch_copy = [&](const Loc& l, int t_) {
        if (!l.ok) return;
        cKE.load(reinterpret_cast<const ET*>(l.base + X::kKE), K, t_);
        cKD.load(reinterpret_cast<const ET*>(l.base + L::kKD), K, t_);
        cTB.load(reinterpret_cast<const ET*>(l.base + L::kTB), kChunk, t_);
        cMS.load(reinterpret_cast<const ET*>(l.base + L::kMS), kChunk, t_);
    };

    // a block's operands in registers: S and dS' (stored transposed: vector e
    // holds keys (e / BV) VE .. +VE-1 of column e % BV), dO rows i (16-byte
    // vectors), and v in the accumulator layout of a wave's tiles
    f32x4 rS[PS], rD[PS], rO[PO];
    // raw, one 32-bit register each (16-bit values are not packed in pairs,
    // which would wait for the request), converted where used
    using RT = typename std::conditional<BF, uint32_t, float>::type;
    RT rv[TW][4];
    auto fetch = [&](const Loc& l, int vb, int t_) {
        if (!l.ok) return;
        const int lane_ = t_ & 63, rt_ = (t_ >> 6) & 3, hv_ = t_ >> 8;
        const int v0 = vb * BV;
        const ET* gS = reinterpret_cast<const ET*>(l.base + X::kS);
        const ET* gDS = reinterpret_cast<const ET*>(l.base + X::kDS);
#pragma unroll
        for (int m = 0; m < PS; ++m) {
            const int e = t_ + m * NT;
            if (NVS % NT == 0 || e < NVS) {
                const int c = e % BV, key = (e / BV) * VE;
                rS[m] = *reinterpret_cast<const f32x4*>(gS + (v0 + c) * K + key);
                rD[m] = *reinterpret_cast<const f32x4*>(gDS + (v0 + c) * K + key);
            }
        }
#pragma unroll
        for (int m = 0; m < PO; ++m) {
            const int e = t_ + m * NT;
            if (NVO % NT == 0 || e < NVO) {
                const int i = e / VPR, c = (e % VPR) * VE;
                rO[m] = i < l.rows ? *reinterpret_cast<const f32x4*>(dOg + ((l.rbase + i) * H + l.h) * V + v0 + c)
                                   : f32x4{0.f, 0.f, 0.f, 0.f};
            }
        }
#pragma unroll
        for (int m = 0; m < TW; ++m) {
            const int ct = hv_ + WPR * m;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = 16 * rt_ + 4 * (lane_ >> 4) + r;
                rv[m][r] = (ct < NCT && i < l.rows)
                               ? static_cast<RT>(vg[((l.rbase + i) * H + l.h) * V + v0 + 16 * ct + (lane_ & 15)])
                               : RT(0);
            }
        }
    };

    auto stage = [&](int t_) {
#pragma unroll
        for (int m = 0; m < PS; ++m) {
            const int e = t_ + m * NT;
            if (NVS % NT == 0 || e < NVS) {
                const int c = e % BV, key = (e / BV) * VE;
                *reinterpret_cast<f32x4*>(&St[c][key]) = rS[m];
                *reinterpret_cast<f32x4*>(&dSt[c][key]) = rD[m];
            }
        }
#pragma unroll
        for (int m = 0; m < PO; ++m) {
            const int e = t_ + m * NT;
            if (NVO % NT == 0 || e < NVO) {
                const int i = e / VPR, c = (e % VPR) * VE;
                *reinterpret_cast<f32x4*>(&dOn[i][c]) = rO[m];
            }
        }
    };

    // the first item: everything requested and waited for here, so that the
    // loop's waits only count requests made one item (or one block) earlier
    int4 mnext = map_entry(blockIdx.x + GS);
    Loc lc = decode(blockIdx.x, map_entry(blockIdx.x));
    fetch_copy(lc, threadIdx.x);
    fetch(lc, 0, threadIdx.x);
    __builtin_amdgcn_s_waitcnt(0);  // vmcnt, expcnt and lgkmcnt all zero

    for (int64_t item = blockIdx.x; item < n_items; item += GS) {
    if (!lc.ok) break;  // items past the last chunk are all empty
    // thread coordinates from an opaque copy of the thread id (keeps the
    // body's LDS addresses from being hoisted out of the item loop)
    int tid = static_cast<int>(threadIdx.x);
    asm volatile("" : "+v"(tid));
    const int t = tid, lane = t & 63, w = t >> 6;
    const int rt = w & 3, hv = w >> 2;  // 16-row tile and column-tile phase of this wave
    const int rows = lc.rows;
    const int h = lc.h;
    const int64_t rbase = lc.rbase;
    uint8_t* base = lc.base;

    cKE.store(&KEn[0][0], LDK, t);
    cKD.store(&KDn[0][0], LDK, t);
    cTB.store(&TBn[0][0], LDC, t);
    cMS.store(&MSn[0][0], LDC, t);
    const Loc ln = decode(item + GS, mnext);
    const int4 mnext2 = map_entry(item + 2 * GS);
    fetch_copy(ln, t);
    asm volatile("" ::: "memory");  // keeps the requests here

    f32x4 aQE[AW], aKE[AW], aKD[AW], aMS[CW], aTB[CW];
#pragma unroll
    for (int c = 0; c < AW; ++c) aQE[c] = aKE[c] = aKD[c] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < CW; ++c) aMS[c] = aTB[c] = f32x4{0.f, 0.f, 0.f, 0.f};
    float dgp[PS][VE];  // dgam partials: keys of the thread's S / dS' vectors, its columns, blocks so far
#pragma unroll
    for (int m = 0; m < PS; ++m)
#pragma unroll
        for (int q = 0; q < VE; ++q) dgp[m][q] = 0.f;
    const int klo = (16 * rt / MM::KS) * MM::KS;

    for (int vb = 0; vb < V / BV; ++vb) {
        const int v0 = vb * BV;
        stage(t);
        // dgam partials from the vectors just staged (bf16 products are exact in fp32)
#pragma unroll
        for (int m = 0; m < PS; ++m) {
            const int e = t + m * NT;
            if (NVS % NT == 0 || e < NVS) {
                if constexpr (BF) {
                    // bf16 pairs: the low half is the earlier key
                    const u32x4_t a = __builtin_bit_cast(u32x4_t, rS[m]), b = __builtin_bit_cast(u32x4_t, rD[m]);
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        dgp[m][2 * q] += __uint_as_float(a[q] << 16) * __uint_as_float(b[q] << 16);
                        dgp[m][2 * q + 1] +=
                            __uint_as_float(a[q] & 0xffff0000u) * __uint_as_float(b[q] & 0xffff0000u);
                    }
                } else {
#pragma unroll
                    for (int q = 0; q < 4; ++q) dgp[m][q] += rS[m][q] * rD[m][q];
                }
            }
        }
        float vcur[TW][4];
#pragma unroll
        for (int m = 0; m < TW; ++m)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                RT x = rv[m][r];
                asm volatile("" : "+v"(x));  // converted here, not right after the request
                if constexpr (BF) vcur[m][r] = bf16_bits_to_f32(static_cast<uint16_t>(x));
                else vcur[m][r] = x;
            }
        {
            // the next block of this item, or the first block of the next
            // item: one request sequence (a branch per case would land them
            // in different registers and copy them, waiting for the data)
            const bool last = vb + 1 == V / BV;
            fetch(last ? ln : lc, last ? 0 : vb + 1, t);
        }
        asm volatile("" ::: "memory");
        __syncthreads();

        // Y = v - KE S and dD = KD dS' + MS^T dO on this wave's tiles
#pragma unroll
        for (int m = 0; m < TW; ++m) {
            const int ct = hv + WPR * m;
            if (ct >= NCT) continue;
            f32x4 pp = {0.f, 0.f, 0.f, 0.f};
            pp = gemm<MM>(&KEn[0][0], LDK, 16 * rt, &St[0][0], LDK, 16 * ct, 0, K, pp, lane);
            f32x4 y;
#pragma unroll
            for (int r = 0; r < 4; ++r) y[r] = vcur[m][r] - pp[r];
            tile_store<MM>(&Yn[0][0], LDB, 16 * rt, 16 * ct, y, lane);
            f32x4 dd = {0.f, 0.f, 0.f, 0.f};
            dd = gemm<MM>(&KDn[0][0], LDK, 16 * rt, &dSt[0][0], LDK, 16 * ct, 0, K, dd, lane);
            for (int k0 = klo; k0 < kChunk; k0 += MM::KS)  // MS^T is upper triangular
                dd = MM::mma(load_kn<MM>(&MSn[0][0], LDC, k0, 16 * rt, lane),
                             load_kn<MM>(&dOn[0][0], LDB, k0, 16 * ct, lane), dd);
            tile_store<MM>(&dDn[0][0], LDB, 16 * rt, 16 * ct, dd, lane);
        }
        __syncthreads();

        // D = TB Y; dY = TB^T dD; dv = dY
#pragma unroll
        for (int m = 0; m < TW; ++m) {
            const int ct = hv + WPR * m;
            if (ct >= NCT) continue;
            f32x4 d = {0.f, 0.f, 0.f, 0.f};
            for (int k0 = 0; k0 < 16 * (rt + 1); k0 += MM::KS)  // TB is lower triangular
                d = MM::mma(load_ap<MM>(&TBn[0][0], LDC, 16 * rt, k0, lane),
                            load_kn<MM>(&Yn[0][0], LDB, k0, 16 * ct, lane), d);
            tile_store<MM>(&Dn[0][0], LDB, 16 * rt, 16 * ct, d, lane);
            f32x4 dy = {0.f, 0.f, 0.f, 0.f};
            for (int k0 = klo; k0 < kChunk; k0 += MM::KS)
                dy = MM::mma(load_kn<MM>(&TBn[0][0], LDC, k0, 16 * rt, lane),
                             load_kn<MM>(&dDn[0][0], LDB, k0, 16 * ct, lane), dy);
            tile_store<MM>(&dYn[0][0], LDB, 16 * rt, 16 * ct, dy, lane);
        }
        __syncthreads();

        // dv = dY, the block's rows from LDS as 16-byte vectors
        for (int e = t; e < kChunk * VPR; e += NT) {
            const int i = e / VPR, c = (e % VPR) * VE;
            if (i < rows)
                *reinterpret_cast<f32x4*>(dvg + ((rbase + i) * H + h) * V + v0 + c) =
                    *reinterpret_cast<const f32x4*>(&dYn[i][c]);
        }

        // V-summed products over this column block (contraction over the block's
        // value columns; S and dS' enter as [v][key] B operands)
#pragma unroll
        for (int m = 0; m < AW; ++m) {
            const int c = hv + WPR * m;
#pragma unroll
            for (int k0 = 0; k0 < BV; k0 += MM::KS) {
                const auto bs = load_kn<MM>(&St[0][0], LDK, k0, 16 * c, lane);
                aQE[m] = MM::mma(load_ap<MM>(&dOn[0][0], LDB, 16 * rt, k0, lane), bs, aQE[m]);
                aKE[m] = MM::mma(load_ap<MM>(&dYn[0][0], LDB, 16 * rt, k0, lane), bs, aKE[m]);
                aKD[m] = MM::mma(load_ap<MM>(&Dn[0][0], LDB, 16 * rt, k0, lane),
                                 load_kn<MM>(&dSt[0][0], LDK, k0, 16 * c, lane), aKD[m]);
            }
        }
#pragma unroll
        for (int m = 0; m < CW; ++m) {
            const int c = hv + WPR * m;
            aMS[m] = gemm<MM>(&dOn[0][0], LDB, 16 * rt, &Dn[0][0], LDB, 16 * c, 0, BV, aMS[m], lane);
            aTB[m] = gemm<MM>(&dDn[0][0], LDB, 16 * rt, &Yn[0][0], LDB, 16 * c, 0, BV, aTB[m], lane);
        }
        __syncthreads();
    }

    ET* gQE = reinterpret_cast<ET*>(base + X::kDQE);
    ET* gKE = reinterpret_cast<ET*>(base + X::kDKE);
    ET* gKD = reinterpret_cast<ET*>(base + X::kDKD);
    ET* gMS = reinterpret_cast<ET*>(base + X::kDMS);
    ET* gTB = reinterpret_cast<ET*>(base + X::kDTB);
#pragma unroll
    for (int m = 0; m < AW; ++m)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = 16 * rt + 4 * (lane >> 4) + r, col = 16 * (hv + WPR * m) + (lane & 15);
            gQE[i * K + col] = MM::from_f32(aQE[m][r]);
            gKE[i * K + col] = MM::from_f32(-aKE[m][r]);
            gKD[i * K + col] = MM::from_f32(aKD[m][r]);
        }
#pragma unroll
    for (int m = 0; m < CW; ++m)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = 16 * rt + 4 * (lane >> 4) + r, col = 16 * (hv + WPR * m) + (lane & 15);
            gMS[i * kChunk + col] = MM::from_f32(aMS[m][r]);
            gTB[i * kChunk + col] = MM::from_f32(aTB[m][r]);
        }
    // dgam: the BV threads of a key vector (aligned lanes of one wave) add
    // their partials, rows of 16 lanes first, then row pairs (the swap of
    // rows 1 and 0, 3 and 2); the thread of column 0 stores the keys
    static_assert(BV == 16 || BV == 32, "a key vector's columns span one or two 16-lane rows");
#pragma unroll
    for (int m = 0; m < PS; ++m) {
        const int e = t + m * NT;
#pragma unroll
        for (int q = 0; q < VE; ++q) {
            float v = row16_sum(dgp[m][q]);
            if constexpr (BV == 32) {
                // the pair's elements go through integer copies: a bit cast
                // applied to an element of the returned vector reads element 0
                const uint32_t u = __builtin_bit_cast(uint32_t, v);
                const auto pr = __builtin_amdgcn_permlane16_swap(u, u, false, false);
                const uint32_t x = pr[0], y = pr[1];
                v = __uint_as_float(x) + __uint_as_float(y);
            }
            dgp[m][q] = v;
        }
        if ((NVS % NT == 0 || e < NVS) && e % BV == 0) {
            float* gd = reinterpret_cast<float*>(base + X::kDGAM) + (e / BV) * VE;
#pragma unroll
            for (int q = 0; q < VE; ++q) gd[q] = dgp[m][q];
        }
    }
    lc = ln;
    mnext = mnext2;
    }  // items
}

// ------------------------------------------------------------------ K-local gradients
template <int K, bool BF>
struct KlocSmem {
    using ET = typename Mma<BF>::ET;
    static constexpr int LDE = K + Mma<BF>::PAD;
    static constexpr int LDC = kChunk + Mma<BF>::PAD;
    ET qh[kChunk][LDE];             // normalised q
    ET kh[kChunk][LDE];             // normalised k
    float G[kChunk][K + 1];         // inclusive cumulative log-decay
    union alignas(16) {
        struct {
            ET Tn[kChunk][LDC];     // T
            ET Tt[kChunk][LDC];     // T^T
            ET dTt[kChunk][LDC];    // (dTB diag(beta))^T
            ET Zn[kChunk][LDC];     // T^T dT
        } mm;
        struct {
            float dM[kChunk][kChunk + 1];  // gradient of the decayed q-k scores
            float dA[kChunk][kChunk + 1];  // gradient of the decayed k-k scores
        } sc;
    } u;
    float beta[kChunk], rq[kChunk], rk[kChunk];
    float dbc[4][kChunk];           // partial sums of dbeta (column part)
    float dbr[kChunk];              // dbeta (row part)
    float red[kThreads / K][K];     // per-part channel partials
    float dots[2][2][kChunk];       // row dot products (q, k) per 64-channel half
    float gpa[kThreads / 64];
};

template <int K, bool BF, int V = K>
__global__ __launch_bounds__(kThreads) void chunk_bwd_klocal_kernel(ChunkParams p, ChunkGrads gr,
                                                                    const int32_t* chunk_off, uint8_t* ws,
                                                                    int64_t slot_bytes) {
    using MM = Mma<BF>;
    using ET = typename MM::ET;
    using IT = typename std::conditional<BF, uint16_t, float>::type;
    using X = BwdExtra<K, BF, V>;
    using SM = KlocSmem<K, BF>;
    constexpr int LDC = SM::LDC;
    constexpr int CPT = K / 4;
    constexpr int NP = kThreads / K;   // row parts in the channel-parallel phases
    constexpr int RPP = kChunk / NP;   // rows per part
    __shared__ __attribute__((aligned(16))) SM s;

    const int H = p.H;
    const int slot = blockIdx.x / H;
    const int h = blockIdx.x % H;
    int n, j;
    int64_t start;
    int len;
    if (!slot_locate(p, chunk_off, slot, n, j, start, len)) return;
    const int rows = min(kChunk, len - j * kChunk);
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    uint8_t* base = ws + (static_cast<int64_t>(slot) * H + h) * slot_bytes;
    const int64_t rbase = start + static_cast<int64_t>(j) * kChunk;
    const float rate = (p.gate_mode == GATE_LOGDECAY) ? 0.f : __expf(p.A_log[h]);

    // ---- 0. prologue again (row-wise), then the cumulative sum (channel-wise)
    {
        const int i = t >> 2, c0 = (t & 3) * CPT;
        const bool valid = i < rows;
        float qv[CPT], kv[CPT], gv[CPT];
        if (valid) {
            const int64_t off = ((rbase + i) * H + h) * K + c0;
            load_row<CPT>(static_cast<const IT*>(p.q) + off, qv);
            load_row<CPT>(static_cast<const IT*>(p.k) + off, kv);
            load_row<CPT>(p.g + off, gv);
        } else {
#pragma unroll
            for (int c = 0; c < CPT; ++c) qv[c] = kv[c] = gv[c] = 0.f;
        }
        float ssq = 0.f, ssk = 0.f;
#pragma unroll
        for (int c = 0; c < CPT; ++c) {
            ssq += qv[c] * qv[c];
            ssk += kv[c] * kv[c];
        }
        ssq += __shfl_xor(ssq, 1, 64);
        ssq += __shfl_xor(ssq, 2, 64);
        ssk += __shfl_xor(ssk, 1, 64);
        ssk += __shfl_xor(ssk, 2, 64);
        float rq = 1.f, rk = 1.f;
        if (p.use_qk_l2norm) {
            rq = rsqrtf(ssq + kL2Eps);
            rk = rsqrtf(ssk + kL2Eps);
        }
        if (!valid) rq = rk = 0.f;
#pragma unroll
        for (int c = 0; c < CPT; ++c) {
            s.qh[i][c0 + c] = MM::from_f32(qv[c] * rq);
            s.kh[i][c0 + c] = MM::from_f32(kv[c] * rk);
            float g = 0.f;
            if (valid) {
                const float bias = p.dt_bias ? p.dt_bias[h * K + c0 + c] : 0.f;
                g = gate_eff(p.gate_mode, gv[c], rate, bias, p.lower_bound);
            }
            s.G[i][c0 + c] = g;
        }
        if ((t & 3) == 0) {
            s.rq[i] = rq;
            s.rk[i] = rk;
            float b = 0.f;
            if (valid) {
                b = p.beta[(rbase + i) * H + h];
                if (p.use_beta_sigmoid) b = sigmoidf_(b);
            }
            s.beta[i] = b;
        }
    }
    __syncthreads();
    const int c = t % K;      // channel of this thread in the channel-parallel phases
    const int hh = t / K;     // row part
    const int r0 = hh * RPP;
    {
        float acc = 0.f;
        for (int r = r0; r < r0 + RPP; ++r) {
            acc += s.G[r][c];
            s.G[r][c] = acc;
        }
        __syncthreads();
        float off = 0.f;
        for (int q = 0; q < hh; ++q) off += s.G[(q + 1) * RPP - 1][c];
        __syncthreads();
        if (hh > 0)
            for (int r = r0; r < r0 + RPP; ++r) s.G[r][c] += off;
    }
    __syncthreads();

    // ---- 1. element-wise terms of QE, KE, KD (channel-parallel, rows r0..r0+RPP)
    const float Glast = s.G[kChunk - 1][c];
    float dqh[RPP], dkh[RPP], dG[RPP];
    float gcp = 0.f;
    {
        const ET* gQE = reinterpret_cast<const ET*>(base + X::kDQE);
        const ET* gKE = reinterpret_cast<const ET*>(base + X::kDKE);
        const ET* gKD = reinterpret_cast<const ET*>(base + X::kDKD);
#pragma unroll
        for (int a = 0; a < RPP; ++a) {
            const int r = r0 + a;
            const float E = __expf(s.G[r][c]);
            const float Ed = __expf(Glast - s.G[r][c]);
            const float q_ = MM::to_f32(s.qh[r][c]), k_ = MM::to_f32(s.kh[r][c]);
            const float dqe = MM::to_f32(gQE[r * K + c]);
            const float dke = MM::to_f32(gKE[r * K + c]);
            const float dkd = MM::to_f32(gKD[r * K + c]);
            const float QE = p.scale * q_ * E, KE = k_ * E, KD = k_ * Ed;
            dqh[a] = p.scale * dqe * E;
            dkh[a] = dke * E + dkd * Ed;
            dG[a] = dqe * QE + dke * KE - dkd * KD;
            gcp += dkd * KD;
        }
    }

    // ---- 2. dA = -T^T (dTB diag(beta)) T^T and the beta terms of TB and A
    {
        const ET* gT = reinterpret_cast<const ET*>(base + X::kT);
        const ET* gTB = reinterpret_cast<const ET*>(base + X::kDTB);
        float part = 0.f;  // column j = t % 64
        for (int e = t; e < kChunk * kChunk; e += kThreads) {
            const int a = e / kChunk, b = e % kChunk;
            const ET tv = gT[e];
            s.u.mm.Tn[a][b] = tv;
            s.u.mm.Tt[b][a] = tv;
            const float dtb = (b <= a) ? MM::to_f32(gTB[e]) : 0.f;
            part += dtb * MM::to_f32(tv);
            s.u.mm.dTt[b][a] = MM::from_f32(dtb * s.beta[b]);
        }
        s.dbc[t >> 6][t & 63] = part;
    }
    __syncthreads();
    {
        f32x4 z[4];
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
            z[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
            z[ct] = gemm<MM>(&s.u.mm.Tt[0][0], LDC, 16 * w, &s.u.mm.dTt[0][0], LDC, 16 * ct, 0, kChunk, z[ct], lane);
        }
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) tile_store<MM>(&s.u.mm.Zn[0][0], LDC, 16 * w, 16 * ct, z[ct], lane);
    }
    __syncthreads();
    f32x4 da[4];
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
        da[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
        da[ct] = gemm<MM>(&s.u.mm.Zn[0][0], LDC, 16 * w, &s.u.mm.Tn[0][0], LDC, 16 * ct, 0, kChunk, da[ct], lane);
    }
    __syncthreads();  // the score buffers below overlay T, Z
    {
        const ET* gAK = reinterpret_cast<const ET*>(base + X::kAK);
        const ET* gMS = reinterpret_cast<const ET*>(base + X::kDMS);
        float rowp[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ct = 0; ct < 4; ++ct)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = 16 * w + 4 * (lane >> 4) + r, jj = 16 * ct + (lane & 15);
                const float dAv = (jj < i) ? -da[ct][r] : 0.f;
                rowp[r] += dAv * MM::to_f32(gAK[i * kChunk + jj]);
                s.u.sc.dA[i][jj] = dAv * s.beta[i];
            }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            float v = rowp[r];
            v += __shfl_xor(v, 1, 64);
            v += __shfl_xor(v, 2, 64);
            v += __shfl_xor(v, 4, 64);
            v += __shfl_xor(v, 8, 64);
            if ((lane & 15) == 0) s.dbr[16 * w + 4 * (lane >> 4) + r] = v;
        }
        for (int e = t; e < kChunk * kChunk; e += kThreads) {
            const int a = e / kChunk, b = e % kChunk;
            s.u.sc.dM[a][b] = (b <= a) ? p.scale * MM::to_f32(gMS[e]) : 0.f;
        }
    }
    __syncthreads();

    // ---- 3. score rule, pairwise, for the q-k (dM) and k-k (dA) scores
#pragma unroll
    for (int a = 0; a < RPP; ++a) {
        const int i = r0 + a;
        const float Gi = s.G[i][c];
        float pq = 0.f, pk = 0.f;
        for (int jj = 0; jj <= i; ++jj) {
            const float e = __expf(Gi - s.G[jj][c]);
            const float kj = MM::to_f32(s.kh[jj][c]) * e;
            pq += s.u.sc.dM[i][jj] * kj;
            pk += s.u.sc.dA[i][jj] * kj;  // zero on the diagonal
        }
        float rq = 0.f, rk = 0.f;
        for (int ii = i; ii < kChunk; ++ii) {
            const float e = __expf(s.G[ii][c] - Gi);
            rq += s.u.sc.dM[ii][i] * MM::to_f32(s.qh[ii][c]) * e;
            rk += s.u.sc.dA[ii][i] * MM::to_f32(s.kh[ii][c]) * e;
        }
        const float q_ = MM::to_f32(s.qh[i][c]), k_ = MM::to_f32(s.kh[i][c]);
        dqh[a] += pq;
        dkh[a] += pk + rq + rk;
        dG[a] += q_ * pq + k_ * pk - k_ * (rq + rk);
    }

    // ---- 4. d(G_last), reverse cumulative sum, gate chain rule
    s.red[hh][c] = gcp;
    __syncthreads();
    if (hh == NP - 1) {
        float tot = 0.f;
#pragma unroll
        for (int q = 0; q < NP; ++q) tot += s.red[q][c];
        const float dgam = reinterpret_cast<const float*>(base + X::kDGAM)[c];
        dG[RPP - 1] += tot + dgam * __expf(Glast);
    }
    __syncthreads();
    {
        float acc = 0.f;
#pragma unroll
        for (int a = RPP - 1; a >= 0; --a) {
            acc += dG[a];
            dG[a] = acc;
        }
        s.red[hh][c] = acc;
    }
    __syncthreads();
    {
        float off = 0.f;
        for (int q = hh + 1; q < NP; ++q) off += s.red[q][c];
        float ddt = 0.f, dal = 0.f;
        const float bias = (p.dt_bias && p.gate_mode != GATE_LOGDECAY) ? p.dt_bias[h * K + c] : 0.f;
#pragma unroll
        for (int a = 0; a < RPP; ++a) {
            const int i = r0 + a;
            const float dge = dG[a] + off;  // gradient of this row's log-decay
            if (i < rows) {
                const int64_t gi = ((rbase + i) * H + h) * K + c;
                float dx = dge;
                if (p.gate_mode != GATE_LOGDECAY) {
                    const float z = p.g[gi] + bias;
                    if (p.gate_mode == GATE_SAFE) {
                        const float sg = sigmoidf_(rate * z);
                        const float base_ = p.lower_bound * sg * (1.f - sg);
                        dx = dge * base_ * rate;
                        dal += dge * base_ * rate * z;
                    } else {
                        float sp, sg;
                        softplus_sigmoid(z, sp, sg);
                        dx = -dge * rate * sg;
                        dal += -dge * rate * sp;
                    }
                    ddt += dx;
                }
                gr.dg[gi] = dx;
            }
        }
        if (p.gate_mode != GATE_LOGDECAY) {
            __syncthreads();
            s.red[hh][c] = ddt;
            dal = wave_sum(dal);
            if (lane == 0) s.gpa[w] = dal;
            __syncthreads();
            float* gp = reinterpret_cast<float*>(base + X::kGP);
            if (hh == 0) {
                float tot = 0.f;
#pragma unroll
                for (int q = 0; q < NP; ++q) tot += s.red[q][c];
                gp[c] = tot;
            }
            if (t == 0) {
                float tot = 0.f;
                for (int q = 0; q < kThreads / 64; ++q) tot += s.gpa[q];
                gp[K] = tot;
            }
        }
    }

    // ---- 5. L2-norm and sigmoid chain rules, stores
    {
        // row dot products q^.dq^ and k^.dk^ over the K channels
        float dq_[RPP], dk_[RPP];
#pragma unroll
        for (int a = 0; a < RPP; ++a) {
            dq_[a] = MM::to_f32(s.qh[r0 + a][c]) * dqh[a];
            dk_[a] = MM::to_f32(s.kh[r0 + a][c]) * dkh[a];
            constexpr int span = K < 64 ? K : 64;
#pragma unroll
            for (int o = 1; o < span; o <<= 1) {
                dq_[a] += __shfl_xor(dq_[a], o, 64);
                dk_[a] += __shfl_xor(dk_[a], o, 64);
            }
        }
        if (K > 64) {
            if ((c & 63) == 0) {
#pragma unroll
                for (int a = 0; a < RPP; ++a) {
                    s.dots[0][c >> 6][r0 + a] = dq_[a];
                    s.dots[1][c >> 6][r0 + a] = dk_[a];
                }
            }
            __syncthreads();
#pragma unroll
            for (int a = 0; a < RPP; ++a) {
                dq_[a] = s.dots[0][0][r0 + a] + s.dots[0][1][r0 + a];
                dk_[a] = s.dots[1][0][r0 + a] + s.dots[1][1][r0 + a];
            }
        }
        IT* dqg = static_cast<IT*>(gr.dq);
        IT* dkg = static_cast<IT*>(gr.dk);
#pragma unroll
        for (int a = 0; a < RPP; ++a) {
            const int i = r0 + a;
            if (i >= rows) continue;
            const int64_t gi = ((rbase + i) * H + h) * K + c;
            float oq = dqh[a], ok = dkh[a];
            if (p.use_qk_l2norm) {
                oq = s.rq[i] * (dqh[a] - MM::to_f32(s.qh[i][c]) * dq_[a]);
                ok = s.rk[i] * (dkh[a] - MM::to_f32(s.kh[i][c]) * dk_[a]);
            }
            Elem<IT>::store(dqg, gi, oq);
            Elem<IT>::store(dkg, gi, ok);
        }
        if (t < kChunk && t < rows) {
            const float db = s.dbc[0][t] + s.dbc[1][t] + s.dbc[2][t] + s.dbc[3][t] + s.dbr[t];
            const float b = s.beta[t];
            gr.dbeta[(rbase + t) * H + h] = p.use_beta_sigmoid ? db * b * (1.f - b) : db;
        }
    }
}

// ------------------------------------------------------------------ K-local gradients, MFMA form
// The same gradients as chunk_bwd_klocal_kernel, for bf16 operands, with the
// score rule on MFMA.  With I the 16-row sub-block of row i, a_i =
// e^(G_i - G_ref(I)) and b_j = e^(G_end(J) - G_j), e^(G_i - G_j) factors as
// a_i * f(J, I) * b_j where f is 1 for adjacent sub-blocks, the decay across
// the sub-blocks in between for J < I - 1, and e^(G_ref(I) - G_end(I)) on the
// diagonal (only where that span is small enough to stay finite; otherwise the
// diagonal sub-block is formed pairwise from G).  Thus
//   P_x = a * sum_J f (dX_IJ (k b)_J),  R = b * sum_I f (dM_IJ^T (q a)_I + dA_IJ^T (k a)_I),
// exact fp32 16 x 16 x 16 products (four fp32 MFMA steps each).
// Each wave takes whole 16-column tiles of dq^, dk^ and dG over all 64 rows
// (a runtime loop when K > 64), so the reverse cumulative sum and the
// d(G_last) term stay inside the wave and each tile's operands are built in
// the wave's own LDS buffer.  With more than one tile per wave, the
// pre-normalisation dq^, dk^ of finished tiles wait in the slot's entry-state
// region (consumed by the V-local kernel) until the row dot products of the
// L2-norm rule are complete.  Workgroups loop over (chunk, head) slots.
template <int K>
struct KlocMfmaSmem {
    using ET = uint16_t;
    static constexpr int LDE = K + 8;
    static constexpr int LDC = kChunk + 8;
    static constexpr int LDG = K + 4;       // G rows: 16-byte aligned, column reads conflict-free
    static constexpr int LDD = kChunk + 4;  // fp32 score-gradient rows, 16-byte aligned
    static constexpr int LDF = kChunk + 4;  // fp32 rows of a tile's score-rule B operand
    // dQE, dKE, dKD staged per wave at K = 64; at K = 32 (two waves per tile)
    // each wave reads its rows' values from the slot where it uses them, and
    // the buffers shrink to a stub, so that two workgroups fit a CU
    static constexpr bool EW_LDS = K / 16 >= 4;
    static constexpr int EWW = EW_LDS ? 4 : 1, EWR = EW_LDS ? kChunk : 1;
    ET qh[kChunk][LDE];             // normalised q
    ET kh[kChunk][LDE];             // normalised k
    float G[kChunk][LDG];           // inclusive cumulative log-decay
    union alignas(16) {
        struct {
            ET Tn[kChunk][LDC];
            ET Tt[kChunk][LDC];
            ET dTt[kChunk][LDC];    // then Z = T^T dT
        } mm;
        struct {
            float dM[kChunk][LDD];  // dMS (lower incl. diagonal), unscaled: exact in bf16
            float dA[kChunk][LDD];  // diag(beta) dA (strictly lower)
        } sc;
    } x;
    float op[4][16][LDF];           // per wave: (k b)^T, (q a)^T or (k a)^T of its tile
    ET ew[EWW][3][EWR][16];         // per wave: the tile's dQE, dKE, dKD
    float P[4][K], invP[4][K];
    float F20[K], F30[K], F31[K];
    float beta[kChunk], rq[kChunk], rk[kChunk];
    float dbc[4][kChunk];
    float dbr[kChunk];
    float dots[2][K / 16][kChunk];  // per-tile row dot products (q^.dq^, k^.dk^)
    float ddt[2][K];                // per half of the rows (K = 32) or whole
    float xch[K / 16][2][16];       // reverse-cumsum terms crossing the halves (K = 32)
    uint32_t lvm[4][2][2][64];      // per lane: level 8 >> lv masks of the P and R rules (level_words)
    float gpa[4];
    int unsafe[4];
};

// fp32 16 x 16 x 16 product for the score rule, as four 16 x 16 x 4 fp32 MFMA
// steps: acc = A[m0 .. m0+15][k0 .. k0+15] * Bt[n0 .. n0+15][k0 .. k0+15]^T.
// The contraction order is permuted so that lane group q supplies the four
// consecutive indices k0 + 4q .. k0 + 4q + 3 (one per step): each lane reads
// its B quad, and its A quad unless TRANS_A, as one 16-byte LDS load.  One
// call spans exactly one 16-row sub-block of the contraction, so the
// per-sub-block factor is applied to the returned tile.  TRANS_A reads A
// transposed (A[k][m]).  Row strides must be multiples of 4 floats.
template <bool TRANS_A>
__device__ __forceinline__ f32x4 mma16_f32(const float* A, int lda, int m0, const float* Bt, int ldb, int n0,
                                           int k0, int lane) {
    const int m = m0 + (lane & 15), n = n0 + (lane & 15), kq = k0 + 4 * (lane >> 4);
    const float4 b4 = *reinterpret_cast<const float4*>(Bt + n * ldb + kq);
    float4 a4;
    if (TRANS_A) {
        a4.x = A[(kq + 0) * lda + m];
        a4.y = A[(kq + 1) * lda + m];
        a4.z = A[(kq + 2) * lda + m];
        a4.w = A[(kq + 3) * lda + m];
    } else {
        a4 = *reinterpret_cast<const float4*>(A + m * lda + kq);
    }
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a4.x, b4.x, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a4.y, b4.y, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a4.z, b4.z, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a4.w, b4.w, acc, 0, 0, 0);
    return acc;
}

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// C += A B over a 16-row contraction with bf16 operands (4 per lane: lane l
// supplies A[l % 16][4 (l / 16) .. + 3] and B[4 (l / 16) .. + 3][l % 16]).
__device__ __forceinline__ f32x4 mfma16x16x16(u32x2 a, u32x2 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a), __builtin_bit_cast(s16x4, b), c,
                                                      0, 0, 0);
}

// Transposing LDS read of four bf16 values (the lo half of load_kn).
__device__ __forceinline__ u32x2 read_tr16(const uint16_t* p) {
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)p));
}

// Four fp32 values as bf16 high parts and bf16 remainders, so that the pair
// holds about 16 bits of each value.
__device__ __forceinline__ void split_hi_lo4(const float (&x)[4], u32x2& hi, u32x2& lo) {
    const bf16x2_t h0 = {static_cast<__bf16>(x[0]), static_cast<__bf16>(x[1])};
    const bf16x2_t h1 = {static_cast<__bf16>(x[2]), static_cast<__bf16>(x[3])};
    const bf16x2_t l0 = {static_cast<__bf16>(x[0] - static_cast<float>(h0[0])),
                         static_cast<__bf16>(x[1] - static_cast<float>(h0[1]))};
    const bf16x2_t l1 = {static_cast<__bf16>(x[2] - static_cast<float>(h1[0])),
                         static_cast<__bf16>(x[3] - static_cast<float>(h1[1]))};
    hi = u32x2{__builtin_bit_cast(uint32_t, h0), __builtin_bit_cast(uint32_t, h1)};
    lo = u32x2{__builtin_bit_cast(uint32_t, l0), __builtin_bit_cast(uint32_t, l1)};
}

typedef float f32x2_t __attribute__((ext_vector_type(2)));

// The products f b0, f b1 as bf16 high parts (one conversion for the pair)
// and bf16 remainders f b - hi, taken of the exact products (fused).
__device__ __forceinline__ void split_prod2(float f, float b0, float b1, uint32_t& hi, uint32_t& lo) {
    hi = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{f * b0, f * b1}, bf16x2_t));
    const float r0 = fmaf(f, b0, -__uint_as_float(hi << 16));
    const float r1 = fmaf(f, b1, -__uint_as_float(hi & 0xffff0000u));
    lo = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{r0, r1}, bf16x2_t));
}

// AND masks over four bf16 entries (two per word) that keep the entries e of
// level_keep(pos, base, h, row_is_later) and clear the others.
__device__ __forceinline__ u32x2 level_words(int pos, int base, int h, bool row_is_later) {
    const unsigned m = level_keep(pos, base, h, row_is_later);
    return u32x2{((m & 1u) ? 0x0000FFFFu : 0u) | ((m & 2u) ? 0xFFFF0000u : 0u),
                 ((m & 4u) ? 0x0000FFFFu : 0u) | ((m & 8u) ? 0xFFFF0000u : 0u)};
}

// Two waves per SIMD are requested from the register allocator: at K = 32 the
// LDS (80.9 KB) holds two workgroups per CU, which the register budget then
// allows too (a few spills, outside the per-slot loops); at K = 64 the LDS
// holds one workgroup and the request has no effect.
template <int K, int V = K>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void chunk_bwd_klocal_mfma_kernel(
    ChunkParams p, ChunkGrads gr, const int32_t* chunk_off, uint8_t* ws, int64_t slot_bytes, int nblk) {
    using MM = Mma<true>;
    using ET = uint16_t;
    using X = BwdExtra<K, true, V>;
    using SM = KlocMfmaSmem<K>;
    constexpr int LDC = SM::LDC;
    constexpr int LDF = SM::LDF;
    constexpr int CPT = K / 4;
    constexpr int NKT = K / 16;
    static_assert(NKT <= 8, "at most two column tiles per wave");
    constexpr bool PARK = NKT > 4;      // each wave owns tiles w and w + 4
    static_assert(!PARK || NKT * 32 * 64 * sizeof(float) <= X::kDQE - X::kS,
                  "parked tiles must fit the state regions");
    __shared__ __attribute__((aligned(16))) SM s;

    const int H = p.H;

    {  // the level masks of every lane, once (they depend on the lane only)
        const int t = threadIdx.x, lane = t & 63, lg = lane >> 4, lc = lane & 15;
        const int lv = t >> 6, hh = 8 >> lv;
        const u32x2 mp = level_words(lc, 4 * lg, hh, true), mr = level_words(lc, 4 * lg, hh, false);
        s.lvm[lv][0][0][lane] = mp[0];
        s.lvm[lv][0][1][lane] = mp[1];
        s.lvm[lv][1][0][lane] = mr[0];
        s.lvm[lv][1][1][lane] = mr[1];
    }
    for (int blk = blockIdx.x; blk < nblk; blk += gridDim.x) {
        // The thread index passes through an empty asm each slot, so the
        // per-lane LDS addresses derived from it are recomputed per slot
        // rather than hoisted out of the loop and kept live across it.
        int t = threadIdx.x;
        asm volatile("" : "+v"(t));
        const int lane = t & 63, w = t >> 6;
        const int lg = lane >> 4, lc = lane & 15;
        const int slot = blk / H;
        const int h = item_head(blk, H, gridDim.x, p.gate_mode != GATE_LOGDECAY);
        int n, j;
        int64_t start;
        int len;
        if (!slot_locate(p, chunk_off, slot, n, j, start, len)) break;  // slots past the last chunk are all empty
        const int rows = min(kChunk, len - j * kChunk);
        uint8_t* base = ws + (static_cast<int64_t>(slot) * H + h) * slot_bytes;
        const int64_t rbase = start + static_cast<int64_t>(j) * kChunk;
        float rate = 0.f;  // e^(A_log[h]), requested in the prologue with the row inputs
        __syncthreads();  // the previous slot is done with the shared buffers

        // ---- 0. prologue (row-wise), cumulative sum, sub-block factors
        {
            const int i = t >> 2, c0 = (t & 3) * CPT;
            const bool valid = i < rows;
            // the gate parameters first, so that the waits for the rows
            // below cover them (one wait, not one per element)
            float bias[CPT];
            if (p.gate_mode != GATE_LOGDECAY && p.dt_bias) {
                load_row<CPT>(p.dt_bias + h * K + c0, bias);
            } else {
#pragma unroll
                for (int c = 0; c < CPT; ++c) bias[c] = 0.f;
            }
            // rate = e^alog is taken at use.  The request is unconditional (a
            // valid word of beta stands in without an in-kernel gate) and its
            // per-lane address (min(t, 0) is 0, which the compiler cannot see)
            // keeps the value in a vector register, so that its wait falls at
            // the use, with the rows'.
            const bool gated = p.gate_mode != GATE_LOGDECAY;
            const float alog = (gated ? p.A_log : p.beta)[(gated ? h : 0) + min(t, 0)];
            float qv[CPT], kv[CPT], gv[CPT];
            float braw = 0.f;
            if (valid) {
                const int64_t off = ((rbase + i) * H + h) * K + c0;
                braw = p.beta[(rbase + i) * H + h];
                load_row<CPT>(static_cast<const uint16_t*>(p.q) + off, qv);
                load_row<CPT>(static_cast<const uint16_t*>(p.k) + off, kv);
                load_row<CPT>(p.g + off, gv);
            } else {
#pragma unroll
                for (int c = 0; c < CPT; ++c) qv[c] = kv[c] = gv[c] = 0.f;
            }
            float ssq = 0.f, ssk = 0.f;
#pragma unroll
            for (int c = 0; c < CPT; ++c) {
                ssq += qv[c] * qv[c];
                ssk += kv[c] * kv[c];
            }
            ssq += __shfl_xor(ssq, 1, 64);
            ssq += __shfl_xor(ssq, 2, 64);
            ssk += __shfl_xor(ssk, 1, 64);
            ssk += __shfl_xor(ssk, 2, 64);
            float rq = 1.f, rk = 1.f;
            if (p.use_qk_l2norm) {
                rq = rsqrtf(ssq + kL2Eps);
                rk = rsqrtf(ssk + kL2Eps);
            }
            if (!valid) rq = rk = 0.f;
            if (p.gate_mode != GATE_LOGDECAY) {
                rate = __expf(alog);
#pragma unroll 4
                for (int c = 0; c < CPT; ++c)
                    gv[c] = valid ? gate_eff(p.gate_mode, gv[c], rate, bias[c], p.lower_bound) : 0.f;
            }
#pragma unroll
            for (int v = 0; v < CPT / 8; ++v) {
                u16x8 uq, uk;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    uq[e] = MM::from_f32(qv[8 * v + e] * rq);
                    uk[e] = MM::from_f32(kv[8 * v + e] * rk);
                }
                *reinterpret_cast<u16x8*>(&s.qh[i][c0 + 8 * v]) = uq;
                *reinterpret_cast<u16x8*>(&s.kh[i][c0 + 8 * v]) = uk;
            }
#pragma unroll
            for (int v = 0; v < CPT / 4; ++v)
                *reinterpret_cast<f32x4*>(&s.G[i][c0 + 4 * v]) =
                    f32x4{gv[4 * v], gv[4 * v + 1], gv[4 * v + 2], gv[4 * v + 3]};
            if ((t & 3) == 0) {
                s.rq[i] = rq;
                s.rk[i] = rk;
                float b = braw;
                if (valid && p.use_beta_sigmoid) b = sigmoidf_(b);
                s.beta[i] = b;
            }
            if (t < 4) s.unsafe[t] = 0;
        }
        __syncthreads();
        {
            constexpr int SEGS = kThreads / K;
            constexpr int SEGLEN = kChunk / SEGS;
            const int c = t % K, sg = t / K;
            float acc = 0.f;
            for (int r = sg * SEGLEN; r < (sg + 1) * SEGLEN; ++r) {
                acc += s.G[r][c];
                s.G[r][c] = acc;
            }
            __syncthreads();
            float off = 0.f;
            for (int q = 0; q < sg; ++q) off += s.G[(q + 1) * SEGLEN - 1][c];
            __syncthreads();
            if (sg > 0)
                for (int r = sg * SEGLEN; r < (sg + 1) * SEGLEN; ++r) s.G[r][c] += off;
        }
        __syncthreads();
        for (int c = t; c < K; c += kThreads) {
#pragma unroll
            for (int I = 0; I < 4; ++I) {
                const float Gref = I == 0 ? 0.f : s.G[kSub * I - 1][c];
                const float span = Gref - s.G[kSub * I + kSub - 1][c];
                s.P[I][c] = __expf(-span);
                s.invP[I][c] = __expf(span);
                if (!(span <= kSpanLimit)) s.unsafe[I] = 1;
            }
            s.F20[c] = s.P[1][c];
            s.F31[c] = s.P[2][c];
            s.F30[c] = s.P[1][c] * s.P[2][c];
        }

        // ---- 1. dA = -T^T (dTB diag(beta)) T^T and the beta terms of TB and A
        // Every global operand of this phase is requested before any is used.
        // Thread t owns column t % 64 of rows t / 64 + 4 e of T, dTB and dMS,
        // and row 16 w + 4 lg + r, column 16 ct + lc of AK (the dA layout).
        ET tv[16], tbv[16], msv[16], akv[16];
        {
            const ET* gT = reinterpret_cast<const ET*>(base + X::kT);
            const ET* gTB = reinterpret_cast<const ET*>(base + X::kDTB);
            const ET* gMS = reinterpret_cast<const ET*>(base + X::kDMS);
            const ET* gAK = reinterpret_cast<const ET*>(base + X::kAK);
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                tv[e] = gT[t + kThreads * e];
                tbv[e] = gTB[t + kThreads * e];
                msv[e] = gMS[t + kThreads * e];
            }
#pragma unroll
            for (int ct = 0; ct < 4; ++ct)
#pragma unroll
                for (int r = 0; r < 4; ++r) akv[4 * ct + r] = gAK[(16 * w + 4 * lg + r) * kChunk + 16 * ct + lc];
        }
        {
            float part = 0.f;  // column t % 64
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int a = (t >> 6) + 4 * e, b = t & 63;
                s.x.mm.Tn[a][b] = tv[e];
                s.x.mm.Tt[b][a] = tv[e];
                const float dtb = (b <= a) ? MM::to_f32(tbv[e]) : 0.f;
                part += dtb * MM::to_f32(tv[e]);
                s.x.mm.dTt[b][a] = MM::from_f32(dtb * s.beta[b]);
            }
            s.dbc[w][t & 63] = part;
        }
        __syncthreads();
        {
            f32x4 z[4];
#pragma unroll
            for (int ct = 0; ct < 4; ++ct) {
                z[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
                z[ct] = gemm<MM>(&s.x.mm.Tt[0][0], LDC, 16 * w, &s.x.mm.dTt[0][0], LDC, 16 * ct, 0, kChunk, z[ct],
                                 lane);
            }
            __syncthreads();  // every wave is done reading dT: Z takes its place
#pragma unroll
            for (int ct = 0; ct < 4; ++ct) tile_store<MM>(&s.x.mm.dTt[0][0], LDC, 16 * w, 16 * ct, z[ct], lane);
        }
        __syncthreads();
        f32x4 da[4];
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
            da[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
            da[ct] = gemm<MM>(&s.x.mm.dTt[0][0], LDC, 16 * w, &s.x.mm.Tn[0][0], LDC, 16 * ct, 0, kChunk, da[ct], lane);
        }
        __syncthreads();  // the score gradients below overlay T and Z
        {
            float rowp[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ct = 0; ct < 4; ++ct)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int i = 16 * w + 4 * lg + r, jj = 16 * ct + lc;
                    const float dAv = (jj < i) ? -da[ct][r] : 0.f;
                    rowp[r] += dAv * MM::to_f32(akv[4 * ct + r]);
                    s.x.sc.dA[i][jj] = dAv * s.beta[i];
                }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float v = rowp[r];
                v += __shfl_xor(v, 1, 64);
                v += __shfl_xor(v, 2, 64);
                v += __shfl_xor(v, 4, 64);
                v += __shfl_xor(v, 8, 64);
                if (lc == 0) s.dbr[16 * w + 4 * lg + r] = v;
            }
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int a = (t >> 6) + 4 * e, b = t & 63;
                s.x.sc.dM[a][b] = (b <= a) ? MM::to_f32(msv[e]) : 0.f;  // the scale is applied to the products
            }
        }
        __syncthreads();

        // ---- 2. per column tile: score rule, element-wise terms, reverse cumsum, gate rule
        // With two column tiles (K = 32) the four waves pair up: wave w takes
        // tile w % 2 and the output rows of half w / 2 (sub-blocks 0-1 or 2-3),
        // so that every SIMD has a share.  The score-rule B operands are built
        // by both waves of a pair; the two terms of the reverse cumulative sum
        // that cross the halves (the upper half's suffix sum at row 32, and the
        // lower half's share of the row-63 term) are exchanged through LDS.
        constexpr int HALVES = NKT < 4 ? 4 / NKT : 1;
        constexpr int IPH = 4 / HALVES;  // output sub-blocks per wave
        static_assert(HALVES == 1 || NKT * HALVES == 4, "tiles x halves = waves");
        const int hf = HALVES > 1 ? w / NKT : 0;
        const int I0 = IPH * hf, I1 = I0 + IPH;
        auto mine = [&](int I) { return HALVES == 1 || (I >= I0 && I < I1); };
        const ET* gQE = reinterpret_cast<const ET*>(base + X::kDQE);
        const ET* gKE = reinterpret_cast<const ET*>(base + X::kDKE);
        const ET* gKD = reinterpret_cast<const ET*>(base + X::kDKD);
        const float* dgam = reinterpret_cast<const float*>(base + X::kDGAM);
        // sub-blocks whose diagonal block takes the level decomposition (bit I)
        const int umask = __builtin_amdgcn_readfirstlane(s.unsafe[0] | s.unsafe[1] << 1 | s.unsafe[2] << 2 |
                                                         s.unsafe[3] << 3);
        auto unsafe = [&](int I) { return (umask >> I & 1) != 0; };
        float (*opw)[LDF] = s.op[w];
        constexpr bool EW_LDS = SM::EW_LDS;
        ET (*eww)[SM::EWR][16] = s.ew[EW_LDS ? w : 0];
        float dal = 0.f;
        f32x4 dq[4], dk[4];
        // per wave and tile, 32 floats per lane (dq^ then dk^), lane-minor
        float* park = reinterpret_cast<float*>(base + X::kS) + w * 2 * 32 * 64 + lane;
#pragma unroll 1
        for (int ct = HALVES > 1 ? w % NKT : w; ct < NKT; ct += 4) {
            const int c = 16 * ct + lc;     // this lane's channel
            // The tile's dQE, dKE, dKD (64 rows x 32 bytes each) are requested
            // now and staged in LDS after the P terms: vector v = lane + 64 hf
            // holds row v / 2, columns 8 (v % 2) .. +7.
            uint4 ewv[6];
            if constexpr (EW_LDS) {
#pragma unroll
                for (int hf = 0; hf < 2; ++hf) {
                    const int v = lane + 64 * hf;
                    const int off = (v >> 1) * K + 16 * ct + 8 * (v & 1);
                    ewv[hf] = *reinterpret_cast<const uint4*>(gQE + off);
                    ewv[2 + hf] = *reinterpret_cast<const uint4*>(gKE + off);
                    ewv[4 + hf] = *reinterpret_cast<const uint4*>(gKD + off);
                }
            }
            // sub-block factors f(J, I) of this lane's column
            float invp[4];
#pragma unroll
            for (int I = 0; I < 4; ++I) invp[I] = unsafe(I) ? 0.f : s.invP[I][c];
            const float f20 = s.F20[c], f30 = s.F30[c], f31 = s.F31[c];
            auto fac = [&](int J, int I) -> float {
                if (J == I) return invp[I];
                if (J == I - 1) return 1.f;
                if (I == 2) return f20;
                return J == 0 ? f30 : f31;
            };
            float Gc[16];  // G of this lane's rows 16 I + 4 lg + r
#pragma unroll
            for (int I = 0; I < 4; ++I)
#pragma unroll
                for (int r = 0; r < 4; ++r) Gc[4 * I + r] = s.G[kSub * I + 4 * lg + r][c];
            f32x4 dG[4];
#pragma unroll
            for (int I = 0; I < 4; ++I) dq[I] = dk[I] = dG[I] = f32x4{0.f, 0.f, 0.f, 0.f};

            // (k b)^T of this tile, b_j = e^(G_end(J) - G_j): lane builds row j = lane
            {
                const int jr = lane, je = kSub * (jr / kSub) + kSub - 1;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float4 g4 = *reinterpret_cast<const float4*>(&s.G[jr][16 * ct + 4 * q]);
                    const float4 e4 = *reinterpret_cast<const float4*>(&s.G[je][16 * ct + 4 * q]);
                    opw[4 * q + 0][jr] = MM::to_f32(s.kh[jr][16 * ct + 4 * q + 0]) * __expf(e4.x - g4.x);
                    opw[4 * q + 1][jr] = MM::to_f32(s.kh[jr][16 * ct + 4 * q + 1]) * __expf(e4.y - g4.y);
                    opw[4 * q + 2][jr] = MM::to_f32(s.kh[jr][16 * ct + 4 * q + 2]) * __expf(e4.z - g4.z);
                    opw[4 * q + 3][jr] = MM::to_f32(s.kh[jr][16 * ct + 4 * q + 3]) * __expf(e4.w - g4.w);
                }
            }
            // P terms: P_x[I] = a_I * sum_J f(J, I) dX_IJ (k b)_J
#pragma unroll
            for (int I = 0; I < 4; ++I) {
                if (!mine(I)) continue;
                f32x4 pq = {0.f, 0.f, 0.f, 0.f}, pk = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int J = 0; J <= I; ++J) {
                    if (J == I && unsafe(I)) continue;  // the level decomposition below
                    const float f = fac(J, I);
                    const f32x4 aq = mma16_f32<false>(&s.x.sc.dM[0][0], SM::LDD, kSub * I, &opw[0][0], LDF, 0,
                                                      kSub * J, lane);
                    const f32x4 ak = mma16_f32<false>(&s.x.sc.dA[0][0], SM::LDD, kSub * I, &opw[0][0], LDF, 0,
                                                      kSub * J, lane);
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        pq[r] += f * aq[r];
                        pk[r] += f * ak[r];
                    }
                }
                const float Gr = I == 0 ? 0.f : s.G[kSub * I - 1][c];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int i = kSub * I + 4 * lg + r;
                    const float a_ = __expf(Gc[4 * I + r] - Gr);
                    const float Pq = a_ * p.scale * pq[r], Pk = a_ * pk[r];
                    dq[I][r] += Pq;
                    dk[I][r] += Pk;
                    dG[I][r] += MM::to_f32(s.qh[i][c]) * Pq + MM::to_f32(s.kh[i][c]) * Pk;
                }
            }
            // stage the element-wise operands (requested at the tile start)
            if constexpr (EW_LDS) {
#pragma unroll
                for (int hf = 0; hf < 2; ++hf) {
                    const int v = lane + 64 * hf;
#pragma unroll
                    for (int a3 = 0; a3 < 3; ++a3)
                        *reinterpret_cast<uint4*>(&eww[a3][v >> 1][8 * (v & 1)]) = ewv[2 * a3 + hf];
                }
            }

            // R terms: (q a)^T against dM, then (k a)^T against dA, a_i = e^(G_i - G_ref(I))
            f32x4 rr[4];
#pragma unroll
            for (int J = 0; J < 4; ++J) rr[J] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
            for (int pass = 0; pass < 2; ++pass) {
                {
                    const int ir = lane, I = ir / kSub;
                    const ET* xr = pass == 0 ? &s.qh[ir][16 * ct] : &s.kh[ir][16 * ct];
                    const float sc = pass == 0 ? p.scale : 1.f;  // dM holds dMS unscaled
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const float4 g4 = *reinterpret_cast<const float4*>(&s.G[ir][16 * ct + 4 * q]);
                        float4 r4 = {0.f, 0.f, 0.f, 0.f};
                        if (I > 0) r4 = *reinterpret_cast<const float4*>(&s.G[kSub * I - 1][16 * ct + 4 * q]);
                        opw[4 * q + 0][ir] = sc * MM::to_f32(xr[4 * q + 0]) * __expf(g4.x - r4.x);
                        opw[4 * q + 1][ir] = sc * MM::to_f32(xr[4 * q + 1]) * __expf(g4.y - r4.y);
                        opw[4 * q + 2][ir] = sc * MM::to_f32(xr[4 * q + 2]) * __expf(g4.z - r4.z);
                        opw[4 * q + 3][ir] = sc * MM::to_f32(xr[4 * q + 3]) * __expf(g4.w - r4.w);
                    }
                }
                const float* dX = pass == 0 ? &s.x.sc.dM[0][0] : &s.x.sc.dA[0][0];
#pragma unroll
                for (int J = 0; J < 4; ++J) {
                    if (!mine(J)) continue;
#pragma unroll
                    for (int I = J; I < 4; ++I) {
                        if (I == J && unsafe(J)) continue;  // the level decomposition below
                        const float f = fac(J, I);
                        const f32x4 acc =
                            mma16_f32<true>(dX, SM::LDD, kSub * J, &opw[0][0], LDF, 0, kSub * I, lane);
#pragma unroll
                        for (int r = 0; r < 4; ++r) rr[J][r] += f * acc[r];
                    }
                }
            }
#pragma unroll
            for (int J = 0; J < 4; ++J) {
                if (!mine(J)) continue;
                const float Ge = s.G[kSub * J + kSub - 1][c];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int i = kSub * J + 4 * lg + r;
                    const float R = __expf(Ge - Gc[4 * J + r]) * rr[J][r];
                    dk[J][r] += R;
                    dG[J][r] -= MM::to_f32(s.kh[i][c]) * R;
                }
            }

            // diagonal sub-blocks too wide to factorise through one reference row:
            // the level decomposition (kda_chunk_common.hpp), every factor <= 1, as
            // 16 x 16 x 16 bf16 products over the block's own 16 rows with the fp32
            // dA and the B values (each lane's own rows of the block) split into
            // bf16 high and low parts (dMS is exact in bf16), the A entries of
            // other levels masked; the diagonal entries directly.  Block values
            // are selected into registers and the contributions added back by
            // selection (no run-time register indexing).
            if (umask) {
#pragma unroll 1
                for (int I = 0; I < 4; ++I) {
                    if (!unsafe(I) || !mine(I)) continue;  // uniform over the wave
                    const int b0 = kSub * I;
                    float gI[4], qI[4], kI[4];
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        gI[r] = I == 0 ? Gc[r] : I == 1 ? Gc[4 + r] : I == 2 ? Gc[8 + r] : Gc[12 + r];
                        qI[r] = MM::to_f32(s.qh[b0 + 4 * lg + r][c]);
                        kI[r] = MM::to_f32(s.kh[b0 + 4 * lg + r][c]);
                    }
                    const float g8 = s.G[b0 + 7][c];
                    const float g4 = s.G[b0 + 4 * (lg & 2) + 3][c];
                    // A operands: rows b0 + lc against contraction rows b0 + 4 lg + e,
                    // and transposed (rows b0 + 4 lg + e of column b0 + lc)
                    float am[4], ak[4], tm[4], tk[4];
                    {
                        const float4 a4 = *reinterpret_cast<const float4*>(&s.x.sc.dM[b0 + lc][b0 + 4 * lg]);
                        const float4 k4 = *reinterpret_cast<const float4*>(&s.x.sc.dA[b0 + lc][b0 + 4 * lg]);
                        am[0] = a4.x; am[1] = a4.y; am[2] = a4.z; am[3] = a4.w;
                        ak[0] = k4.x; ak[1] = k4.y; ak[2] = k4.z; ak[3] = k4.w;
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            tm[e] = s.x.sc.dM[b0 + 4 * lg + e][b0 + lc];
                            tk[e] = s.x.sc.dA[b0 + 4 * lg + e][b0 + lc];
                        }
                    }
                    u32x2 amh, aml, akh, akl, tmh, tml, tkh, tkl;
                    split_hi_lo4(am, amh, aml);  // aml and tml are zero
                    split_hi_lo4(ak, akh, akl);
                    split_hi_lo4(tm, tmh, tml);
                    split_hi_lo4(tk, tkh, tkl);
                    f32x4 dqI = {0.f, 0.f, 0.f, 0.f}, dkI = dqI, dGI = dqI;
#pragma unroll 1
                    for (int lv = 0; lv < 4; ++lv) {
                        const int hh = 8 >> lv;
                        float f[4];
                        bool later[4];
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const float gref = hh == 8 ? g8 : hh == 4 ? g4 : hh == 2 ? gI[1] : gI[r & 2];
                            later[r] = (4 * lg + r) & hh;
                            f[r] = __expf(later[r] ? gI[r] - gref : gref - gI[r]);
                        }
                        const u32x2 wP = {s.lvm[lv][0][0][lane], s.lvm[lv][0][1][lane]};
                        const u32x2 wR = {s.lvm[lv][1][0][lane], s.lvm[lv][1][1][lane]};
                        float b4[4];
                        u32x2 bh, bl;
                        // P terms (the scale is applied to the q products)
#pragma unroll
                        for (int r = 0; r < 4; ++r) b4[r] = later[r] ? 0.f : kI[r] * f[r];
                        split_hi_lo4(b4, bh, bl);
                        f32x4 pq = {0.f, 0.f, 0.f, 0.f}, pk = {0.f, 0.f, 0.f, 0.f};
                        pq = mfma16x16x16(amh & wP, bh, pq);
                        pq = mfma16x16x16(amh & wP, bl, pq);
                        pk = mfma16x16x16(akh & wP, bh, pk);
                        pk = mfma16x16x16(akh & wP, bl, pk);
                        pk = mfma16x16x16(akl & wP, bh, pk);
                        // R terms: q against dM, then k against dA
                        f32x4 rr = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int r = 0; r < 4; ++r) b4[r] = later[r] ? p.scale * qI[r] * f[r] : 0.f;
                        split_hi_lo4(b4, bh, bl);
                        rr = mfma16x16x16(tmh & wR, bh, rr);
                        rr = mfma16x16x16(tmh & wR, bl, rr);
#pragma unroll
                        for (int r = 0; r < 4; ++r) b4[r] = later[r] ? kI[r] * f[r] : 0.f;
                        split_hi_lo4(b4, bh, bl);
                        rr = mfma16x16x16(tkh & wR, bh, rr);
                        rr = mfma16x16x16(tkh & wR, bl, rr);
                        rr = mfma16x16x16(tkl & wR, bh, rr);
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const float Pq = later[r] ? f[r] * p.scale * pq[r] : 0.f;
                            const float Pk = later[r] ? f[r] * pk[r] : 0.f;
                            const float R = later[r] ? 0.f : f[r] * rr[r];
                            dqI[r] += Pq;
                            dkI[r] += Pk + R;
                            dGI[r] += qI[r] * Pq + kI[r] * (Pk - R);
                        }
                    }
                    // the diagonal entries (no decay): dM_ii enters both rules and
                    // their dG terms cancel; dA is strictly lower
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int i = b0 + 4 * lg + r;
                        const float dmii = p.scale * s.x.sc.dM[i][i];
                        dqI[r] += dmii * kI[r];
                        dkI[r] += dmii * qI[r];
                    }
#pragma unroll
                    for (int II = 0; II < 4; ++II)
                        if (II == I) {
                            dq[II] += dqI;
                            dk[II] += dkI;
                            dG[II] += dGI;
                        }
                }
            }

            // element-wise terms of QE, KE, KD and d(G_last)
            const float Glast = s.G[kChunk - 1][c];
            float colp = 0.f;
#pragma unroll
            for (int I = 0; I < 4; ++I) {
                if (!mine(I)) continue;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int i = kSub * I + 4 * lg + r;
                    const float Gi = Gc[4 * I + r];
                    const float E = __expf(Gi), Ed = __expf(Glast - Gi);
                    const float q_ = MM::to_f32(s.qh[i][c]), k_ = MM::to_f32(s.kh[i][c]);
                    float dqe, dke, dkd;
                    if constexpr (EW_LDS) {
                        dqe = MM::to_f32(eww[0][i][lc]);
                        dke = MM::to_f32(eww[1][i][lc]);
                        dkd = MM::to_f32(eww[2][i][lc]);
                    } else {
                        dqe = MM::to_f32(gQE[i * K + c]);
                        dke = MM::to_f32(gKE[i * K + c]);
                        dkd = MM::to_f32(gKD[i * K + c]);
                    }
                    const float KD = k_ * Ed;
                    dq[I][r] += p.scale * dqe * E;
                    dk[I][r] += dke * E + dkd * Ed;
                    dG[I][r] += dqe * p.scale * q_ * E + dke * k_ * E - dkd * KD;
                    colp += dkd * KD;
                }
            }
            colp += __shfl_xor(colp, 16, 64);
            colp += __shfl_xor(colp, 32, 64);
            // the row-63 term: this wave's share of sum(dKD * KD) and d(G_last)
            // (the lower half's share reaches every row as a constant below)
            if (I1 == 4 && lg == 3) dG[3][3] += colp + dgam[c] * __expf(Glast);

            // reverse cumulative sum over the 64 rows of this column
            float carry = 0.f;
#pragma unroll
            for (int I = 3; I >= 0; --I) {
                if (!mine(I)) continue;
                dG[I][2] += dG[I][3];
                dG[I][1] += dG[I][2];
                dG[I][0] += dG[I][1];
                const float own = dG[I][0];
                const float up1 = __shfl(own, (lane + 16) & 63, 64);
                const float up2 = __shfl(own, (lane + 32) & 63, 64);
                const float up3 = __shfl(own, (lane + 48) & 63, 64);
                float add = carry;
                if (lg < 3) add += up1;
                if (lg < 2) add += up2;
                if (lg < 1) add += up3;
#pragma unroll
                for (int r = 0; r < 4; ++r) dG[I][r] += add;
                carry = __shfl(dG[I][0], lc, 64);  // suffix sum from row 16 I
            }
            if constexpr (HALVES > 1) {
                // the lower half adds the upper half's suffix sum at row 32 and
                // its own row-63 share; the upper half adds the lower half's share
                if (lg == 0) s.xch[ct][hf][lc] = hf == 0 ? colp : carry;
                __syncthreads();  // every wave of the workgroup is here once
                const float add = hf == 0 ? colp + s.xch[ct][1][lc] : s.xch[ct][0][lc];
#pragma unroll
                for (int I = 0; I < 4; ++I)
                    if (mine(I)) dG[I] += f32x4{add, add, add, add};
            }

            // gate chain rule.  Every gate input is requested before the first
            // d(gate) store (loads and stores share one in-order counter, so a
            // load issued behind a store would also wait for that store), each
            // sub-block's at its use: a request one sub-block ahead would be
            // waited for at once and spilled at this register budget.  dG
            // becomes d(gate input) in place.
            const float bias = (p.dt_bias && p.gate_mode != GATE_LOGDECAY) ? p.dt_bias[h * K + c] : 0.f;
            float ddt = 0.f;
            if (p.gate_mode != GATE_LOGDECAY) {
                float zc[4];
                auto zload = [&](int I, float (&z)[4]) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int i = kSub * I + 4 * lg + r;
                        const int ic = i < rows ? i : rows - 1;  // a slot holds at least one row
                        z[r] = p.g[((rbase + ic) * H + h) * K + c];
                    }
                };
#pragma unroll
                for (int I = 0; I < 4; ++I) {
                    if (!mine(I)) continue;
                    zload(I, zc);
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int i = kSub * I + 4 * lg + r;
                        const float dge = dG[I][r];
                        const float z = zc[r] + bias;
                        float dx, da;
                        if (p.gate_mode == GATE_SAFE) {
                            const float sg = sigmoidf_(rate * z);
                            const float b_ = p.lower_bound * sg * (1.f - sg);
                            dx = dge * b_ * rate;
                            da = dx * z;
                        } else {
                            float sp, sg;
                            softplus_sigmoid(z, sp, sg);
                            dx = -dge * rate * sg;
                            da = -dge * rate * sp;
                        }
                        if (i < rows) {
                            ddt += dx;
                            dal += da;
                        }
                        dG[I][r] = dx;
                    }
                }
            }
#pragma unroll
            for (int I = 0; I < 4; ++I) {
                if (!mine(I)) continue;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int i = kSub * I + 4 * lg + r;
                    if (i < rows) gr.dg[((rbase + i) * H + h) * K + c] = dG[I][r];
                }
            }
            ddt += __shfl_xor(ddt, 16, 64);
            ddt += __shfl_xor(ddt, 32, 64);
            if (lg == 0) s.ddt[hf][c] = ddt;

            // row dot products of the L2-norm rule
#pragma unroll
            for (int I = 0; I < 4; ++I) {
                if (!mine(I)) continue;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int i = kSub * I + 4 * lg + r;
                    float vq = MM::to_f32(s.qh[i][c]) * dq[I][r];
                    float vk = MM::to_f32(s.kh[i][c]) * dk[I][r];
#pragma unroll
                    for (int o = 1; o < 16; o <<= 1) {
                        vq += __shfl_xor(vq, o, 64);
                        vk += __shfl_xor(vk, o, 64);
                    }
                    if (lc == 0) {
                        s.dots[0][ct][i] = vq;
                        s.dots[1][ct][i] = vk;
                    }
                }
            }
            // with two tiles per wave, the tile's dq^, dk^ wait for the row
            // dot products in this lane's own strip of the slot's state
            // regions (read by the V-local kernel, free now), coalesced across
            // the wave; a single tile stays in registers
            if (PARK) {
                float* pk = park + ((ct - w) / 4) * 32 * 64;
#pragma unroll
                for (int I = 0; I < 4; ++I)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        pk[(4 * I + r) * 64] = dq[I][r];
                        pk[(16 + 4 * I + r) * 64] = dk[I][r];
                    }
            }
        }

        // ---- 3. L2-norm and sigmoid chain rules, gate shares, stores
        __syncthreads();  // dots and ddt are complete
        if (t < 2 * kChunk) {  // row totals of the dot products, kept in tile slot 0
            const int i = t & (kChunk - 1), which = t / kChunk;
            float acc = 0.f;
#pragma unroll
            for (int q = 0; q < NKT; ++q) acc += s.dots[which][q][i];
            s.dots[which][0][i] = acc;
        }
        __syncthreads();
        {
            uint16_t* dqg = static_cast<uint16_t*>(gr.dq);
            uint16_t* dkg = static_cast<uint16_t*>(gr.dk);
            auto store_tile = [&](int ct, const f32x4* tq, const f32x4* tk) {
                const int c = 16 * ct + lc;
#pragma unroll
                for (int I = 0; I < 4; ++I)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int i = kSub * I + 4 * lg + r;
                        if (i >= rows || !mine(I)) continue;
                        const float dotq = s.dots[0][0][i], dotk = s.dots[1][0][i];
                        float oq = tq[I][r], ok = tk[I][r];
                        if (p.use_qk_l2norm) {
                            oq = s.rq[i] * (oq - MM::to_f32(s.qh[i][c]) * dotq);
                            ok = s.rk[i] * (ok - MM::to_f32(s.kh[i][c]) * dotk);
                        }
                        const int64_t gi = ((rbase + i) * H + h) * K + c;
                        dqg[gi] = f32_to_bf16_bits(oq);
                        dkg[gi] = f32_to_bf16_bits(ok);
                    }
            };
            if (!PARK) {
                if (HALVES > 1) store_tile(w % NKT, dq, dk);
                else if (w < NKT) store_tile(w, dq, dk);
            } else
#pragma unroll 1
            for (int ct = w; ct < NKT; ct += 4) {
                const float* pk = park + ((ct - w) / 4) * 32 * 64;
                f32x4 tq[4], tk[4];
#pragma unroll
                for (int I = 0; I < 4; ++I)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        tq[I][r] = pk[(4 * I + r) * 64];
                        tk[I][r] = pk[(16 + 4 * I + r) * 64];
                    }
                store_tile(ct, tq, tk);
            }
        }
        if (t < kChunk && t < rows) {
            const float db = s.dbc[0][t] + s.dbc[1][t] + s.dbc[2][t] + s.dbc[3][t] + s.dbr[t];
            const float b = s.beta[t];
            gr.dbeta[(rbase + t) * H + h] = p.use_beta_sigmoid ? db * b * (1.f - b) : db;
        }
        if (p.gate_mode != GATE_LOGDECAY) {
            dal = wave_sum(dal);
            if (lane == 0) s.gpa[w] = dal;
            __syncthreads();
            float* gp = reinterpret_cast<float*>(base + X::kGP);
            for (int cc = t; cc < K; cc += kThreads) gp[cc] = HALVES > 1 ? s.ddt[0][cc] + s.ddt[1][cc] : s.ddt[0][cc];
            if (t == 0) gp[K] = s.gpa[0] + s.gpa[1] + s.gpa[2] + s.gpa[3];
        }
    }
}

// ------------------------------------------------------------------ K-local gradients, 8 waves (K = 128)
// The computation of chunk_bwd_klocal_mfma_kernel with one 16-column tile per
// wave: 8 waves, two per SIMD, so that one wave's LDS and memory latency
// overlaps another's work.  In the score-rule products (contraction order
// permuted as in mma16_f32) each lane's four B values per step lie in its own
// rows and column of the tile, so the B operands (k b), (q a), (k a) are
// formed in registers; only the fp32 score gradients dM and dA are shared
// through LDS.  The tile's dQE, dKE, dKD are requested at the start of the
// slot and staged one array at a time through a 2 KB buffer per wave.
struct KlocW8Smem {
    using ET = uint16_t;
    static constexpr int K = 128;
    static constexpr int LDE = K + 8;
    static constexpr int LDC = kChunk + 8;
    static constexpr int LDG = K + 4;
    static constexpr int LDD = kChunk + 4;
    ET qh[kChunk][LDE];
    ET kh[kChunk][LDE];
    float G[kChunk][LDG];
    union alignas(16) {
        struct {
            ET Tn[kChunk][LDC];
            ET Tt[kChunk][LDC];
            ET dTt[kChunk][LDC];
            ET Zn[kChunk][LDC];
        } mm;
        struct {
            ET dM[kChunk][LDC];   // dMS (lower incl. diagonal) as stored: bf16, exact
            ET dA[kChunk][LDC];   // diag(beta) dA (strictly lower), bf16 high part
            ET dAl[kChunk][LDC];  // and the bf16 remainder, so that hi + lo holds 16 bits
        } sc;
        struct {
            ET dq[kChunk][LDE];     // the slot's dq and dk rows on their way out
            ET dk[kChunk][LDE];
        } out;
    } x;
    ET ew[8][kChunk][16];
    float invP[4][K];
    float F20[K], F30[K], F31[K];
    float beta[kChunk], rq[kChunk], rk[kChunk];
    float dbc[8][kChunk];
    float dbr[2][kChunk];
    float dots[2][8][kChunk];
    float ddt[K];
    float gpa[8];
    int unsafe[4];
};

// fp32 16 x 16 x 16 product accumulated into acc, with the lane's four B
// values given (step st uses b[st], the B element at contraction index
// k0 + 4 (lane / 16) + st); TRANS_A reads A[k][m] instead of A[m][k].
template <bool TRANS_A>
__device__ __forceinline__ f32x4 mma16_f32_rb_acc(const float* A, int lda, int m0, const float* b, int k0, int lane,
                                                  f32x4 acc) {
    const int m = m0 + (lane & 15), kq = k0 + 4 * (lane >> 4);
    float4 a4;
    if (TRANS_A) {
        a4.x = A[(kq + 0) * lda + m];
        a4.y = A[(kq + 1) * lda + m];
        a4.z = A[(kq + 2) * lda + m];
        a4.w = A[(kq + 3) * lda + m];
    } else {
        a4 = *reinterpret_cast<const float4*>(A + m * lda + kq);
    }
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a4.x, b[0], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a4.y, b[1], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a4.z, b[2], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a4.w, b[3], acc, 0, 0, 0);
    return acc;
}

constexpr int kKlocW8Threads = 512;

__global__ __launch_bounds__(kKlocW8Threads) void chunk_bwd_klocal_w8_kernel(ChunkParams p, ChunkGrads gr,
                                                                            const int32_t* chunk_off, uint8_t* ws,
                                                                            int64_t slot_bytes, int nblk) {
    using MM = Mma<true>;
    using ET = uint16_t;
    constexpr int K = 128;
    using X = BwdExtra<K, true>;
    using SM = KlocW8Smem;
    constexpr int NT = kKlocW8Threads;
    constexpr int NW = NT / 64;
    constexpr int LDC = SM::LDC;
    constexpr int LDD = SM::LDD;
    constexpr int TPR = NT / kChunk;  // threads per row in the prologue
    constexpr int CPT = K / TPR;
    static_assert(NW * 16 == K, "one 16-column tile per wave");
    __shared__ __attribute__((aligned(16))) SM s;

    const int H = p.H;

    for (int blk = blockIdx.x; blk < nblk; blk += gridDim.x) {
        // The thread index passes through an empty asm each slot, so the
        // per-lane LDS addresses derived from it are recomputed per slot
        // rather than hoisted out of the loop (where they would be spilled).
        int t = threadIdx.x;
        asm volatile("" : "+v"(t));
        const int lane = t & 63, w = t >> 6;
        const int lg = lane >> 4, lc = lane & 15;
        const int c = 16 * w + lc;  // this lane's channel in the tile phase
        const int slot = blk / H;
        const int h = item_head(blk, H, gridDim.x, p.gate_mode != GATE_LOGDECAY);
        int n, j;
        int64_t start;
        int len;
        if (!slot_locate(p, chunk_off, slot, n, j, start, len)) break;  // slots past the last chunk are all empty
        const int rows = min(kChunk, len - j * kChunk);
        uint8_t* base = ws + (static_cast<int64_t>(slot) * H + h) * slot_bytes;
        const int64_t rbase = start + static_cast<int64_t>(j) * kChunk;
        float rate = 0.f;  // e^(A_log[h]), requested in the prologue with the row inputs
        __syncthreads();  // the previous slot is done with the shared buffers

        // stage 1's operands are requested first, so that their latency
        // overlaps the prologue's
        const int rt = w & 3, ch = w >> 2;  // this wave's dA tiles: (rt, ch) and (rt, ch + 2)
        ET tv[8], tbv[8], msv[8], akv[8];
        {
            const ET* gT = reinterpret_cast<const ET*>(base + X::kT);
            const ET* gTB = reinterpret_cast<const ET*>(base + X::kDTB);
            const ET* gMS = reinterpret_cast<const ET*>(base + X::kDMS);
            const ET* gAK = reinterpret_cast<const ET*>(base + X::kAK);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                tv[e] = gT[t + NT * e];
                tbv[e] = gTB[t + NT * e];
                msv[e] = gMS[t + NT * e];
            }
#pragma unroll
            for (int m = 0; m < 2; ++m)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    akv[4 * m + r] = gAK[(16 * rt + 4 * lg + r) * kChunk + 16 * (ch + 2 * m) + lc];
        }

        // ---- 0. prologue (row-wise), cumulative sum, sub-block factors
        {
            const int i = t / TPR, c0 = (t % TPR) * CPT;
            const bool valid = i < rows;
            // the gate parameters first, so that the waits for the rows
            // below cover them (one wait, not one per element)
            float bias[CPT];
            if (p.gate_mode != GATE_LOGDECAY && p.dt_bias) {
                load_row<CPT>(p.dt_bias + h * K + c0, bias);
            } else {
#pragma unroll
                for (int cc = 0; cc < CPT; ++cc) bias[cc] = 0.f;
            }
            // rate = e^alog is taken at use.  The request is unconditional (a
            // valid word of beta stands in without an in-kernel gate) and its
            // per-lane address (min(t, 0) is 0, which the compiler cannot see)
            // keeps the value in a vector register, so that its wait falls at
            // the use, with the rows'.
            const bool gated = p.gate_mode != GATE_LOGDECAY;
            const float alog = (gated ? p.A_log : p.beta)[(gated ? h : 0) + min(t, 0)];
            float qv[CPT], kv[CPT], gv[CPT];
            float braw = 0.f;
            if (valid) {
                const int64_t off = ((rbase + i) * H + h) * K + c0;
                braw = p.beta[(rbase + i) * H + h];
                load_row<CPT>(static_cast<const uint16_t*>(p.q) + off, qv);
                load_row<CPT>(static_cast<const uint16_t*>(p.k) + off, kv);
                load_row<CPT>(p.g + off, gv);
            } else {
#pragma unroll
                for (int cc = 0; cc < CPT; ++cc) qv[cc] = kv[cc] = gv[cc] = 0.f;
            }
            float ssq = 0.f, ssk = 0.f;
#pragma unroll
            for (int cc = 0; cc < CPT; ++cc) {
                ssq += qv[cc] * qv[cc];
                ssk += kv[cc] * kv[cc];
            }
#pragma unroll
            for (int o = 1; o < TPR; o <<= 1) {
                ssq += __shfl_xor(ssq, o, 64);
                ssk += __shfl_xor(ssk, o, 64);
            }
            float rq = 1.f, rk = 1.f;
            if (p.use_qk_l2norm) {
                rq = rsqrtf(ssq + kL2Eps);
                rk = rsqrtf(ssk + kL2Eps);
            }
            if (!valid) rq = rk = 0.f;
            if (p.gate_mode != GATE_LOGDECAY) {
                rate = __expf(alog);
#pragma unroll 4
                for (int cc = 0; cc < CPT; ++cc)
                    gv[cc] = valid ? gate_eff(p.gate_mode, gv[cc], rate, bias[cc], p.lower_bound) : 0.f;
            }
#pragma unroll
            for (int v = 0; v < CPT / 8; ++v) {
                u16x8 uq, uk;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    uq[e] = MM::from_f32(qv[8 * v + e] * rq);
                    uk[e] = MM::from_f32(kv[8 * v + e] * rk);
                }
                *reinterpret_cast<u16x8*>(&s.qh[i][c0 + 8 * v]) = uq;
                *reinterpret_cast<u16x8*>(&s.kh[i][c0 + 8 * v]) = uk;
            }
#pragma unroll
            for (int v = 0; v < CPT / 4; ++v)
                *reinterpret_cast<f32x4*>(&s.G[i][c0 + 4 * v]) =
                    f32x4{gv[4 * v], gv[4 * v + 1], gv[4 * v + 2], gv[4 * v + 3]};
            if (t % TPR == 0) {
                s.rq[i] = rq;
                s.rk[i] = rk;
                s.beta[i] = (valid && p.use_beta_sigmoid) ? sigmoidf_(braw) : braw;
            }
            if (t < 4) s.unsafe[t] = 0;
        }
        __syncthreads();
        {
            constexpr int SEGS = NT / K;
            constexpr int SEGLEN = kChunk / SEGS;
            const int cc = t % K, sg = t / K;
            float acc = 0.f;
            for (int r = sg * SEGLEN; r < (sg + 1) * SEGLEN; ++r) {
                acc += s.G[r][cc];
                s.G[r][cc] = acc;
            }
            __syncthreads();
            float off = 0.f;
            for (int q = 0; q < sg; ++q) off += s.G[(q + 1) * SEGLEN - 1][cc];
            __syncthreads();
            if (sg > 0)
                for (int r = sg * SEGLEN; r < (sg + 1) * SEGLEN; ++r) s.G[r][cc] += off;
        }
        __syncthreads();
        if (t < K) {
            float P[4];
#pragma unroll
            for (int I = 0; I < 4; ++I) {
                const float Gref = I == 0 ? 0.f : s.G[kSub * I - 1][t];
                const float span = Gref - s.G[kSub * I + kSub - 1][t];
                P[I] = __expf(-span);
                s.invP[I][t] = __expf(span);
                if (!(span <= kSpanLimit)) s.unsafe[I] = 1;
            }
            s.F20[t] = P[1];
            s.F31[t] = P[2];
            s.F30[t] = P[1] * P[2];
        }

        // ---- 1. dA = -T^T (dTB diag(beta)) T^T and the beta terms of TB and A.
        // Thread t owns column t % 64 of rows t / 64 + 8 e of T, dTB and dMS;
        // wave w owns the dA tiles (w % 4, w / 4) and (w % 4, w / 4 + 2).
        {
            float part = 0.f;  // column t % 64
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int a = (t >> 6) + 8 * e, b = t & 63;
                s.x.mm.Tn[a][b] = tv[e];
                s.x.mm.Tt[b][a] = tv[e];
                const float dtb = (b <= a) ? MM::to_f32(tbv[e]) : 0.f;
                part += dtb * MM::to_f32(tv[e]);
                s.x.mm.dTt[b][a] = MM::from_f32(dtb * s.beta[b]);
            }
            s.dbc[w][t & 63] = part;
        }
        __syncthreads();
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            f32x4 z = {0.f, 0.f, 0.f, 0.f};
            z = gemm<MM>(&s.x.mm.Tt[0][0], LDC, 16 * rt, &s.x.mm.dTt[0][0], LDC, 16 * (ch + 2 * m), 0, kChunk, z, lane);
            tile_store<MM>(&s.x.mm.Zn[0][0], LDC, 16 * rt, 16 * (ch + 2 * m), z, lane);
        }
        __syncthreads();
        f32x4 da[2];
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            da[m] = f32x4{0.f, 0.f, 0.f, 0.f};
            da[m] = gemm<MM>(&s.x.mm.Zn[0][0], LDC, 16 * rt, &s.x.mm.Tn[0][0], LDC, 16 * (ch + 2 * m), 0, kChunk,
                             da[m], lane);
        }
        __syncthreads();  // the score gradients below overlay T and Z
        {
            float rowp[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int m = 0; m < 2; ++m)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int i = 16 * rt + 4 * lg + r, jj = 16 * (ch + 2 * m) + lc;
                    const float dAv = (jj < i) ? -da[m][r] : 0.f;
                    rowp[r] += dAv * MM::to_f32(akv[4 * m + r]);
                    const float x_ = dAv * s.beta[i];
                    const ET hi = MM::from_f32(x_);
                    s.x.sc.dA[i][jj] = hi;
                    s.x.sc.dAl[i][jj] = MM::from_f32(x_ - MM::to_f32(hi));
                }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float v = rowp[r];
                v += __shfl_xor(v, 1, 64);
                v += __shfl_xor(v, 2, 64);
                v += __shfl_xor(v, 4, 64);
                v += __shfl_xor(v, 8, 64);
                if (lc == 0) s.dbr[ch][16 * rt + 4 * lg + r] = v;
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int a = (t >> 6) + 8 * e, b = t & 63;
                s.x.sc.dM[a][b] = (b <= a) ? msv[e] : ET(0);  // the scale is applied to the products
            }
        }
        __syncthreads();

        // ---- 2. this wave's column tile: score rule, element-wise terms, reverse cumsum, gate rule
        // this wave's tile of dQE, dKE, dKD (64 rows x 32 bytes each), requested at
        // the start of the tile phase: vector v = lane + 64 hf holds row v / 2, columns 8 (v % 2) .. +7
        uint4 ewv[6];
        {
            const ET* gQE = reinterpret_cast<const ET*>(base + X::kDQE);
            const ET* gKE = reinterpret_cast<const ET*>(base + X::kDKE);
            const ET* gKD = reinterpret_cast<const ET*>(base + X::kDKD);
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                const int v = lane + 64 * hf;
                const int off = (v >> 1) * K + 16 * w + 8 * (v & 1);
                ewv[hf] = *reinterpret_cast<const uint4*>(gQE + off);
                ewv[2 + hf] = *reinterpret_cast<const uint4*>(gKE + off);
                ewv[4 + hf] = *reinterpret_cast<const uint4*>(gKD + off);
            }
        }

        float dal = 0.f;
        f32x4 dq[4], dk[4];
        {
            float Gc[16], qo[16], ko[16];  // the lane's rows 16 I + 4 lg + r of column c
#pragma unroll
            for (int I = 0; I < 4; ++I)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int i = kSub * I + 4 * lg + r;
                    Gc[4 * I + r] = s.G[i][c];
                    qo[4 * I + r] = MM::to_f32(s.qh[i][c]);
                    ko[4 * I + r] = MM::to_f32(s.kh[i][c]);
                }
            // sub-blocks whose diagonal block takes the level decomposition (bit I)
            const int umask = __builtin_amdgcn_readfirstlane(s.unsafe[0] | s.unsafe[1] << 1 | s.unsafe[2] << 2 |
                                                             s.unsafe[3] << 3);
            auto unsafe = [&](int I) { return (umask >> I & 1) != 0; };
            float Ge[4], Gr[4], invp[4];
#pragma unroll
            for (int I = 0; I < 4; ++I) {
                Ge[I] = s.G[kSub * I + kSub - 1][c];
                Gr[I] = I == 0 ? 0.f : s.G[kSub * I - 1][c];
                invp[I] = unsafe(I) ? 0.f : s.invP[I][c];
            }
            const float f20 = s.F20[c], f30 = s.F30[c], f31 = s.F31[c];
            auto fac = [&](int J, int I) -> float {
                if (J == I) return invp[I];
                if (J == I - 1) return 1.f;
                if (I == 2) return f20;
                return J == 0 ? f30 : f31;
            };
            f32x4 dG[4];
#pragma unroll
            for (int I = 0; I < 4; ++I) dq[I] = dk[I] = dG[I] = f32x4{0.f, 0.f, 0.f, 0.f};

            // P terms: P_x[I] = a_I * sum_J f(J, I) dX_IJ (k b)_J,  b_j = e^(G_end(J) - G_j)
            float bv[16];
#pragma unroll
            for (int J = 0; J < 4; ++J)
#pragma unroll
                for (int r = 0; r < 4; ++r) bv[4 * J + r] = ko[4 * J + r] * __expf(Ge[J] - Gc[4 * J + r]);
            // f(J, I) scales column c of every term, so it is folded into the
            // B values and the sums over J accumulate in the MFMA.  bf16 products
            // with two sub-blocks J, J + 1 per contraction step (contraction order
            // of load_ap): the lane's B values are its own rows of both.  B is
            // split into bf16 high and low parts, and so is dA (dMS is exact in
            // bf16), so that the products keep about 16 bits of their operands.
            // A half whose sub-block lies outside the product (has0 / has1
            // false, known at compile time) is zero without arithmetic.
            auto pair_b = [&](float f0, int b0, bool has0, float f1, int b1, bool has1, MM::Frag& hi,
                              MM::Frag& lo) {
                uint32_t h[4] = {0u, 0u, 0u, 0u}, l[4] = {0u, 0u, 0u, 0u};
                if (has0) {
                    split_prod2(f0, bv[4 * b0], bv[4 * b0 + 1], h[0], l[0]);
                    split_prod2(f0, bv[4 * b0 + 2], bv[4 * b0 + 3], h[1], l[1]);
                }
                if (has1) {
                    split_prod2(f1, bv[4 * b1], bv[4 * b1 + 1], h[2], l[2]);
                    split_prod2(f1, bv[4 * b1 + 2], bv[4 * b1 + 3], h[3], l[3]);
                }
                hi = __builtin_bit_cast(MM::Frag, u32x4_t{h[0], h[1], h[2], h[3]});
                lo = __builtin_bit_cast(MM::Frag, u32x4_t{l[0], l[1], l[2], l[3]});
            };
            f32x4 pq[4], pk[4];
#pragma unroll
            for (int I = 0; I < 4; ++I) pq[I] = pk[I] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int I = 0; I < 4; ++I)
#pragma unroll
                for (int Jp = 0; Jp <= I; Jp += 2) {
                    if (Jp == I && unsafe(I)) continue;  // only the diagonal block, taken below
                    MM::Frag bh, bl;
                    pair_b(fac(Jp, I), Jp, true, Jp + 1 <= I ? fac(Jp + 1, I) : 0.f, Jp + 1, Jp + 1 <= I, bh, bl);
                    const auto am = load_ap<MM>(&s.x.sc.dM[0][0], LDC, kSub * I, kSub * Jp, lane);
                    const auto ah = load_ap<MM>(&s.x.sc.dA[0][0], LDC, kSub * I, kSub * Jp, lane);
                    const auto al = load_ap<MM>(&s.x.sc.dAl[0][0], LDC, kSub * I, kSub * Jp, lane);
                    pq[I] = MM::mma(am, bh, pq[I]);
                    pq[I] = MM::mma(am, bl, pq[I]);
                    pk[I] = MM::mma(ah, bh, pk[I]);
                    pk[I] = MM::mma(ah, bl, pk[I]);
                    pk[I] = MM::mma(al, bh, pk[I]);
                }
#pragma unroll
            for (int I = 0; I < 4; ++I)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float a_ = __expf(Gc[4 * I + r] - Gr[I]);
                    const float Pq = a_ * p.scale * pq[I][r], Pk = a_ * pk[I][r];
                    dq[I][r] += Pq;
                    dk[I][r] += Pk;
                    dG[I][r] += qo[4 * I + r] * Pq + ko[4 * I + r] * Pk;
                }

            // R terms: (q a) against dM, then (k a) against dA, a_i = e^(G_i - G_ref(I))
            f32x4 rr[4];
#pragma unroll
            for (int J = 0; J < 4; ++J) rr[J] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
                for (int I = 0; I < 4; ++I)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        bv[4 * I + r] = (pass == 0 ? p.scale * qo[4 * I + r] : ko[4 * I + r]) *
                                        __expf(Gc[4 * I + r] - Gr[I]);
                // A = dX^T (transposing read); sub-blocks I < J contribute nothing
#pragma unroll
                for (int J = 0; J < 4; ++J)
#pragma unroll
                    for (int Ip = 0; Ip < 4; Ip += 2) {
                        if (Ip + 1 < J) continue;
                        if (Ip + 1 == J && unsafe(J)) continue;  // only the diagonal block, taken below
                        MM::Frag bh, bl;
                        pair_b(Ip >= J ? fac(J, Ip) : 0.f, Ip, Ip >= J, fac(J, Ip + 1), Ip + 1, true, bh, bl);
                        if (pass == 0) {
                            const auto am = load_kn<MM>(&s.x.sc.dM[0][0], LDC, kSub * Ip, kSub * J, lane);
                            rr[J] = MM::mma(am, bh, rr[J]);
                            rr[J] = MM::mma(am, bl, rr[J]);
                        } else {
                            const auto ah = load_kn<MM>(&s.x.sc.dA[0][0], LDC, kSub * Ip, kSub * J, lane);
                            const auto al = load_kn<MM>(&s.x.sc.dAl[0][0], LDC, kSub * Ip, kSub * J, lane);
                            rr[J] = MM::mma(ah, bh, rr[J]);
                            rr[J] = MM::mma(ah, bl, rr[J]);
                            rr[J] = MM::mma(al, bh, rr[J]);
                        }
                    }
            }
#pragma unroll
            for (int J = 0; J < 4; ++J)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float R = __expf(Ge[J] - Gc[4 * J + r]) * rr[J][r];
                    dk[J][r] += R;
                    dG[J][r] -= ko[4 * J + r] * R;
                }

            // diagonal sub-blocks too wide to factorise through one reference row:
            // the level decomposition (kda_chunk_common.hpp), every factor <= 1, as
            // 16 x 16 x 16 bf16 products over the block's own 16 rows (each lane's
            // four B values are its own rows of the block), with the A entries of
            // other levels masked; the diagonal entries directly.  One copy of the
            // code serves every block: the block's register values are selected
            // in and its contributions added back by selection, so that no
            // register array is indexed at run time.
            if (umask) {
#pragma unroll 1
                for (int I = 0; I < 4; ++I) {
                    if (!unsafe(I)) continue;  // uniform over the workgroup
                    float gI[4], qI[4], kI[4];
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        gI[r] = I == 0 ? Gc[r] : I == 1 ? Gc[4 + r] : I == 2 ? Gc[8 + r] : Gc[12 + r];
                        qI[r] = I == 0 ? qo[r] : I == 1 ? qo[4 + r] : I == 2 ? qo[8 + r] : qo[12 + r];
                        kI[r] = I == 0 ? ko[r] : I == 1 ? ko[4 + r] : I == 2 ? ko[8 + r] : ko[12 + r];
                    }
                    const int b0 = kSub * I;
                    const float g8 = s.G[b0 + 7][c];
                    const float g4 = s.G[b0 + 4 * (lg & 2) + 3][c];
                    // A operands of the block: rows b0 + lc against contraction rows
                    // b0 + 4 lg + e, and the transposed reads (rows b0 + 4 lg + e of
                    // column b0 + lc) for the column-side rule
                    const u32x2 am0 = *reinterpret_cast<const u32x2*>(&s.x.sc.dM[b0 + lc][b0 + 4 * lg]);
                    const u32x2 ah0 = *reinterpret_cast<const u32x2*>(&s.x.sc.dA[b0 + lc][b0 + 4 * lg]);
                    const u32x2 al0 = *reinterpret_cast<const u32x2*>(&s.x.sc.dAl[b0 + lc][b0 + 4 * lg]);
                    const int tro = (b0 + 4 * lg + (lc >> 2)) * LDC + b0 + 4 * (lc & 3);
                    const u32x2 tm0 = read_tr16(&s.x.sc.dM[0][0] + tro);
                    const u32x2 th0 = read_tr16(&s.x.sc.dA[0][0] + tro);
                    const u32x2 tl0 = read_tr16(&s.x.sc.dAl[0][0] + tro);
                    f32x4 dqI = {0.f, 0.f, 0.f, 0.f}, dkI = dqI, dGI = dqI;
#pragma unroll
                    for (int lv = 0; lv < 4; ++lv) {
                        const int hh = 8 >> lv;
                        float f[4];
                        bool later[4];
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const float gref = hh == 8 ? g8 : hh == 4 ? g4 : hh == 2 ? gI[1] : gI[r & 2];
                            later[r] = (4 * lg + r) & hh;
                            f[r] = __expf(later[r] ? gI[r] - gref : gref - gI[r]);
                        }
                        const u32x2 wP = level_words(lc, 4 * lg, hh, true);
                        const u32x2 wR = level_words(lc, 4 * lg, hh, false);
                        // P terms: rows i (later half) against columns j (earlier half)
                        float b4[4];
#pragma unroll
                        for (int r = 0; r < 4; ++r) b4[r] = later[r] ? 0.f : kI[r] * f[r];
                        u32x2 bh, bl;
                        split_hi_lo4(b4, bh, bl);
                        const u32x2 am = am0 & wP, ah = ah0 & wP, al = al0 & wP;
                        f32x4 pq = {0.f, 0.f, 0.f, 0.f}, pk = {0.f, 0.f, 0.f, 0.f};
                        pq = mfma16x16x16(am, bh, pq);
                        pq = mfma16x16x16(am, bl, pq);
                        pk = mfma16x16x16(ah, bh, pk);
                        pk = mfma16x16x16(ah, bl, pk);
                        pk = mfma16x16x16(al, bh, pk);
                        // R terms: columns j (earlier half) against rows i (later half)
                        f32x4 rr = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int r = 0; r < 4; ++r) b4[r] = later[r] ? p.scale * qI[r] * f[r] : 0.f;
                        split_hi_lo4(b4, bh, bl);
                        const u32x2 tm = tm0 & wR;
                        rr = mfma16x16x16(tm, bh, rr);
                        rr = mfma16x16x16(tm, bl, rr);
#pragma unroll
                        for (int r = 0; r < 4; ++r) b4[r] = later[r] ? kI[r] * f[r] : 0.f;
                        split_hi_lo4(b4, bh, bl);
                        const u32x2 th = th0 & wR, tl = tl0 & wR;
                        rr = mfma16x16x16(th, bh, rr);
                        rr = mfma16x16x16(th, bl, rr);
                        rr = mfma16x16x16(tl, bh, rr);
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const float Pq = later[r] ? f[r] * p.scale * pq[r] : 0.f;
                            const float Pk = later[r] ? f[r] * pk[r] : 0.f;
                            const float R = later[r] ? 0.f : f[r] * rr[r];
                            dqI[r] += Pq;
                            dkI[r] += Pk + R;
                            dGI[r] += qI[r] * Pq + kI[r] * (Pk - R);
                        }
                    }
                    // the diagonal entries (no decay): dM_ii enters both rules and
                    // their dG terms cancel; dA is strictly lower
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int i = b0 + 4 * lg + r;
                        const float dmii = p.scale * MM::to_f32(s.x.sc.dM[i][i]);
                        dqI[r] += dmii * kI[r];
                        dkI[r] += dmii * qI[r];
                    }
#pragma unroll
                    for (int II = 0; II < 4; ++II)
                        if (II == I) {
                            dq[II] += dqI;
                            dk[II] += dkI;
                            dG[II] += dGI;
                        }
                }
            }

            // element-wise terms of QE, KE, KD and d(G_last); the operands pass
            // through the wave's 2 KB buffer one array at a time
            const float Glast = s.G[kChunk - 1][c];
            float E[16];
#pragma unroll
            for (int q = 0; q < 16; ++q) E[q] = __expf(Gc[q]);
            ET (*eww)[16] = s.ew[w];
            float colp = 0.f;
#pragma unroll
            for (int a3 = 0; a3 < 3; ++a3) {
#pragma unroll
                for (int hf = 0; hf < 2; ++hf) {
                    const int v = lane + 64 * hf;
                    *reinterpret_cast<uint4*>(&eww[v >> 1][8 * (v & 1)]) = ewv[2 * a3 + hf];
                }
#pragma unroll
                for (int I = 0; I < 4; ++I)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int q = 4 * I + r;
                        const float x_ = MM::to_f32(eww[kSub * I + 4 * lg + r][lc]);
                        if (a3 == 0) {
                            dq[I][r] += p.scale * x_ * E[q];
                            dG[I][r] += x_ * p.scale * qo[q] * E[q];
                        } else if (a3 == 1) {
                            dk[I][r] += x_ * E[q];
                            dG[I][r] += x_ * ko[q] * E[q];
                        } else {
                            const float Ed = __expf(Glast - Gc[q]);
                            const float KD = ko[q] * Ed;
                            dk[I][r] += x_ * Ed;
                            dG[I][r] -= x_ * KD;
                            colp += x_ * KD;
                        }
                    }
            }
            colp += __shfl_xor(colp, 16, 64);
            colp += __shfl_xor(colp, 32, 64);
            if (lg == 3)
                dG[3][3] += colp + reinterpret_cast<const float*>(base + X::kDGAM)[c] * __expf(Glast);

            // reverse cumulative sum over the 64 rows of this column
            float carry = 0.f;
#pragma unroll
            for (int I = 3; I >= 0; --I) {
                dG[I][2] += dG[I][3];
                dG[I][1] += dG[I][2];
                dG[I][0] += dG[I][1];
                const float own = dG[I][0];
                const float up1 = __shfl(own, (lane + 16) & 63, 64);
                const float up2 = __shfl(own, (lane + 32) & 63, 64);
                const float up3 = __shfl(own, (lane + 48) & 63, 64);
                float add = carry;
                if (lg < 3) add += up1;
                if (lg < 2) add += up2;
                if (lg < 1) add += up3;
#pragma unroll
                for (int r = 0; r < 4; ++r) dG[I][r] += add;
                carry = __shfl(dG[I][0], lc, 64);  // suffix sum from row 16 I
            }

            // gate chain rule.  Every gate input is requested before the first
            // d(gate) store, one sub-block ahead of its use: loads and stores
            // share one in-order counter, so a load issued behind a store would
            // also wait for that store.  dG becomes d(gate input) in place.
            const float bias = (p.dt_bias && p.gate_mode != GATE_LOGDECAY) ? p.dt_bias[h * K + c] : 0.f;
            float ddt = 0.f;
            if (p.gate_mode != GATE_LOGDECAY) {
                float zc[4], zn[4];
                auto zload = [&](int I, float (&z)[4]) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int i = kSub * I + 4 * lg + r;
                        const int ic = i < rows ? i : rows - 1;  // a slot holds at least one row
                        z[r] = p.g[((rbase + ic) * H + h) * K + c];
                    }
                };
                zload(0, zc);
#pragma unroll
                for (int I = 0; I < 4; ++I) {
                    if (I < 3) zload(I + 1, zn);
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int i = kSub * I + 4 * lg + r;
                        const float dge = dG[I][r];
                        const float z = zc[r] + bias;
                        float dx, da;
                        if (p.gate_mode == GATE_SAFE) {
                            const float sg = sigmoidf_(rate * z);
                            const float b_ = p.lower_bound * sg * (1.f - sg);
                            dx = dge * b_ * rate;
                            da = dx * z;
                        } else {
                            float sp, sg;
                            softplus_sigmoid(z, sp, sg);
                            dx = -dge * rate * sg;
                            da = -dge * rate * sp;
                        }
                        if (i < rows) {
                            ddt += dx;
                            dal += da;
                        }
                        dG[I][r] = dx;
                    }
                    if (I < 3) {
#pragma unroll
                        for (int r = 0; r < 4; ++r) zc[r] = zn[r];
                    }
                }
            }
#pragma unroll
            for (int I = 0; I < 4; ++I)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int i = kSub * I + 4 * lg + r;
                    if (i < rows) gr.dg[((rbase + i) * H + h) * K + c] = dG[I][r];
                }
            ddt += __shfl_xor(ddt, 16, 64);
            ddt += __shfl_xor(ddt, 32, 64);
            if (lg == 0) s.ddt[c] = ddt;

            // row dot products of the L2-norm rule
#pragma unroll
            for (int I = 0; I < 4; ++I)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float vq = row16_sum(qo[4 * I + r] * dq[I][r]);
                    const float vk = row16_sum(ko[4 * I + r] * dk[I][r]);
                    if (lc == 0) {
                        s.dots[0][w][kSub * I + 4 * lg + r] = vq;
                        s.dots[1][w][kSub * I + 4 * lg + r] = vk;
                    }
                }
        }

        // ---- 3. L2-norm and sigmoid chain rules, gate shares, stores
        __syncthreads();  // dots and ddt are complete
        if (t < 2 * kChunk) {  // row totals of the dot products, kept in tile slot 0
            const int i = t & (kChunk - 1), which = t / kChunk;
            float acc = 0.f;
#pragma unroll
            for (int q = 0; q < NW; ++q) acc += s.dots[which][q][i];
            s.dots[which][0][i] = acc;
        }
        __syncthreads();
        {
            // dq and dk through LDS (the union's score gradients are done),
            // then out as 16-byte row segments
#pragma unroll
            for (int I = 0; I < 4; ++I)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int i = kSub * I + 4 * lg + r;
                    float oq = dq[I][r], ok = dk[I][r];
                    if (p.use_qk_l2norm) {
                        oq = s.rq[i] * (oq - MM::to_f32(s.qh[i][c]) * s.dots[0][0][i]);
                        ok = s.rk[i] * (ok - MM::to_f32(s.kh[i][c]) * s.dots[1][0][i]);
                    }
                    s.x.out.dq[i][c] = f32_to_bf16_bits(oq);
                    s.x.out.dk[i][c] = f32_to_bf16_bits(ok);
                }
            __syncthreads();
            uint16_t* dqg = static_cast<uint16_t*>(gr.dq);
            uint16_t* dkg = static_cast<uint16_t*>(gr.dk);
            constexpr int SEG = K / 8;  // 16-byte segments per row
#pragma unroll
            for (int m = 0; m < kChunk * SEG / NT; ++m) {
                const int e = t + NT * m, i = e / SEG, c8 = 8 * (e % SEG);
                if (i < rows) {
                    const int64_t gi = ((rbase + i) * H + h) * K + c8;
                    *reinterpret_cast<u16x8*>(dqg + gi) = *reinterpret_cast<const u16x8*>(&s.x.out.dq[i][c8]);
                    *reinterpret_cast<u16x8*>(dkg + gi) = *reinterpret_cast<const u16x8*>(&s.x.out.dk[i][c8]);
                }
            }
        }
        if (t < kChunk && t < rows) {
            float db = s.dbr[0][t] + s.dbr[1][t];
#pragma unroll
            for (int q = 0; q < NW; ++q) db += s.dbc[q][t];
            const float b = s.beta[t];
            gr.dbeta[(rbase + t) * H + h] = p.use_beta_sigmoid ? db * b * (1.f - b) : db;
        }
        if (p.gate_mode != GATE_LOGDECAY) {
            dal = wave_sum(dal);
            if (lane == 0) s.gpa[w] = dal;
            __syncthreads();
            float* gp = reinterpret_cast<float*>(base + X::kGP);
            for (int cc = t; cc < K; cc += NT) gp[cc] = s.ddt[cc];
            if (t == 0) {
                float a = 0.f;
#pragma unroll
                for (int q = 0; q < NW; ++q) a += s.gpa[q];
                gp[K] = a;
            }
        }
    }
}

// d(A_log) and d(dt_bias): deterministic sums of the per-chunk shares.  One
// workgroup per head; thread (slot lane sl, column lane cl) sums the slots
// sl, sl + SL, ... of its columns with eight requests in flight, and the SL
// slot lanes' sums are added in a fixed order, so results are run-to-run
// identical without atomics.  At K <= 64 the K + 1 columns take 64 column
// lanes, so that 16 slot lanes share the slots.
constexpr int kGateReduceThreads = 1024;
template <int K>
__global__ __launch_bounds__(kGateReduceThreads) void gate_param_reduce_kernel(ChunkParams p, ChunkGrads gr,
                                                                              const int32_t* chunk_off,
                                                                              const uint8_t* ws, int64_t slot_bytes,
                                                                              size_t gp_off) {
    constexpr int CL = K >= 128 ? 128 : 64;      // column lanes
    constexpr int SL = kGateReduceThreads / CL;  // slot lanes
    constexpr int NCOL = K + 1;                  // K d(dt_bias) shares and the d(A_log) share
    constexpr int CPL = (NCOL + CL - 1) / CL;    // columns per column lane
    __shared__ float part[SL][CPL * CL];
    const int h = blockIdx.x;
    const int H = p.H;
    const int nslots = p.cu_seqlens ? min(chunk_off[p.N], p.total_chunks_bound) : p.N * n_chunks(p.T);
    const int cl = threadIdx.x % CL, sl = threadIdx.x / CL;
#pragma unroll
    for (int m = 0; m < CPL; ++m) {
        const int c = cl + CL * m;
        float acc = 0.f;
        if (c < NCOL) {
            auto share = [&](int s_) {
                return reinterpret_cast<const float*>(ws + (static_cast<int64_t>(s_) * H + h) * slot_bytes + gp_off)[c];
            };
            int s_ = sl;
            for (; s_ + 7 * SL < nslots; s_ += 8 * SL) {
                float a[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) a[u] = share(s_ + u * SL);
#pragma unroll
                for (int u = 0; u < 8; ++u) acc += a[u];
            }
            for (; s_ < nslots; s_ += SL) acc += share(s_);
        }
        part[sl][c] = acc;
    }
    __syncthreads();
    for (int c = threadIdx.x; c < NCOL; c += kGateReduceThreads) {
        float tot = 0.f;
#pragma unroll
        for (int q = 0; q < SL; ++q) tot += part[q][c];
        if (c < K) {
            if (gr.ddt_bias) gr.ddt_bias[h * K + c] = tot;
        } else if (gr.dA_log) {
            gr.dA_log[h] = tot;
        }
    }
}

// ------------------------------------------------------------------ host side
template <int K, bool BF, int V = K>
static size_t bwd_bytes(const ChunkParams& p) {
    return chunk_off_bytes(p) + static_cast<size_t>(p.total_chunks_bound) * p.H * BwdExtra<K, BF, V>::kBytes;
}

size_t chunk_bwd_workspace(const ChunkParams& p) {
    if (p.K == 32 && p.V == 64) return p.bf16 ? bwd_bytes<32, true, 64>(p) : bwd_bytes<32, false, 64>(p);
    if (p.K != p.V) return 0;
    switch (p.K) {
        case 32: return p.bf16 ? bwd_bytes<32, true>(p) : bwd_bytes<32, false>(p);
        case 64: return p.bf16 ? bwd_bytes<64, true>(p) : bwd_bytes<64, false>(p);
        case 128: return p.bf16 ? bwd_bytes<128, true>(p) : 0;
        default: return 0;
    }
}

template <int K, int BV, bool BF, int V = K>
static hipError_t run_bwd(const ChunkParams& p, const ChunkGrads& gr, void* ws, hipStream_t st, int stage) {
    using X = BwdExtra<K, BF, V>;
    uint8_t* w8 = static_cast<uint8_t*>(ws);
    int32_t* chunk_off = reinterpret_cast<int32_t*>(w8);
    uint8_t* slots = w8 + chunk_off_bytes(p);
    const int64_t sb = static_cast<int64_t>(X::kBytes);
    const int64_t nblk = static_cast<int64_t>(p.total_chunks_bound) * p.H;
    const int cgrid = chain_grid(p.N * p.H, V / BV);
    // with p.keep the forward has already done stages 0 and 1
    auto want = [stage, &p](int s) { return (stage < 0 || stage == s) && !(p.keep && s < 2); };
    if (want(0)) {
        if (p.cu_seqlens)
            hipLaunchKernelGGL(plan_chunks_kernel, dim3(1), dim3(kPlanThreads), 0, st, p.cu_seqlens, p.N, p.T, chunk_off,
                               p.total_chunks_bound);
        if (nblk > 0)
            hipLaunchKernelGGL((chunk_prep_kernel<K, BF, true, V>), dim3(prep_grid<K, BF, true, V>(nblk)),
                               dim3(prep_threads(K)), 0, st, p, chunk_off, slots, sb, nblk);
    }
    if (want(1) && cgrid > 0) {
        if constexpr (K == 128 && V == 128 && BF) {
            if (state_pc_bv(p.N * p.H) == 32)
                hipLaunchKernelGGL((chunk_state_fwd_pc_kernel<true, false, 32>), dim3(cgrid),
                                   dim3(state_pc_threads(32)), 0, st, p, chunk_off, slots, sb);
            else
                hipLaunchKernelGGL((chunk_state_fwd_pc_kernel<true, false, 64>), dim3(chain_grid(p.N * p.H, 2)),
                                   dim3(state_pc_threads(64)), 0, st, p, chunk_off, slots, sb);
        } else if (cgrid <= kPersistentGrid)  // few chains: 8 waves per chain (see the forward)
            hipLaunchKernelGGL((chunk_state_fwd_kernel<K, V, BV, BF, true, false, 512>), dim3(cgrid), dim3(512), 0,
                               st, p, chunk_off, slots, sb);
        else
            hipLaunchKernelGGL((chunk_state_fwd_kernel<K, V, BV, BF, true, false>), dim3(cgrid), dim3(kThreads), 0,
                               st, p, chunk_off, slots, sb);
    }
    if (want(2) && cgrid > 0) {
        if constexpr (K == 128 && V == 128 && BF) {
            if (state_pc_bv(p.N * p.H) == 32)
                hipLaunchKernelGGL(chunk_state_bwd_pc_kernel<32>, dim3(cgrid), dim3(state_pc_threads(32)), 0, st, p, gr,
                                   chunk_off, slots, sb);
            else
                hipLaunchKernelGGL(chunk_state_bwd_pc_kernel<64>, dim3(chain_grid(p.N * p.H, 2)),
                                   dim3(state_pc_threads(64)), 0, st, p, gr, chunk_off, slots, sb);
        } else
            hipLaunchKernelGGL((chunk_state_bwd_kernel<K, V, BV, BF>), dim3(cgrid), dim3(kThreads), 0, st, p, gr,
                               chunk_off, slots, sb);
    }
    if (want(3) && nblk > 0)
        hipLaunchKernelGGL((chunk_bwd_vlocal_kernel<K, V, BV, BF>), dim3(vlocal_grid(nblk)),
                           dim3(vlocal_threads(BF)), 0, st, p, gr, chunk_off, slots, sb, nblk);
    if (want(4)) {
        if (nblk > 0) {
            if constexpr (BF && K == 128 && V == 128)
                hipLaunchKernelGGL(chunk_bwd_klocal_w8_kernel,
                                   dim3(static_cast<unsigned>(nblk < kPersistentGrid ? nblk : kPersistentGrid)),
                                   dim3(kKlocW8Threads), 0, st, p, gr, chunk_off, slots, sb, static_cast<int>(nblk));
            else if constexpr (BF) {
                // at K = 32 the shared buffers fit two workgroups per CU
                constexpr int grid = sizeof(KlocMfmaSmem<K>) <= 80 * 1024 ? 2 * kPersistentGrid : kPersistentGrid;
                hipLaunchKernelGGL((chunk_bwd_klocal_mfma_kernel<K, V>),
                                   dim3(static_cast<unsigned>(nblk < grid ? nblk : grid)), dim3(kThreads), 0, st, p,
                                   gr, chunk_off, slots, sb, static_cast<int>(nblk));
            }
            else
                hipLaunchKernelGGL((chunk_bwd_klocal_kernel<K, BF, V>), dim3(static_cast<unsigned>(nblk)),
                                   dim3(kThreads), 0, st, p, gr, chunk_off, slots, sb);
        }
        if (p.gate_mode != GATE_LOGDECAY && (gr.dA_log || gr.ddt_bias))
            hipLaunchKernelGGL((gate_param_reduce_kernel<K>), dim3(p.H), dim3(kGateReduceThreads), 0, st, p, gr,
                               chunk_off, slots, sb,
                               X::kGP);
    }
    return hipGetLastError();
}

hipError_t launch_chunk_bwd(const ChunkParams& p, const ChunkGrads& gr, void* ws, hipStream_t st, int stage) {
    if (p.K == 32 && p.V == 64)
        return p.bf16 ? run_bwd<32, 32, true, 64>(p, gr, ws, st, stage) : run_bwd<32, 16, false, 64>(p, gr, ws, st, stage);
    if (p.K != p.V) return hipErrorInvalidValue;
    switch (p.K) {
        case 32: return p.bf16 ? run_bwd<32, 32, true>(p, gr, ws, st, stage) : run_bwd<32, 16, false>(p, gr, ws, st, stage);
        case 64: return p.bf16 ? run_bwd<64, 32, true>(p, gr, ws, st, stage) : run_bwd<64, 16, false>(p, gr, ws, st, stage);
        case 128: return p.bf16 ? run_bwd<128, 32, true>(p, gr, ws, st, stage) : hipErrorInvalidValue;
        default: return hipErrorInvalidValue;
    }
}

}  // namespace kda
