// hh_wide.hip -- chunked Hedgehog linear attention on the CDNA4 matrix cores (bf16 in, fp32 state).
//
// What is computed (paper-graph-ui walkthrough of "The Hedgehog & the
// Porcupine", section 2 Eq. 2 and section 3.4 "Complexity Analysis"):
//     y_i = phi(q_i)^T S_i / phi(q_i)^T z_i,   S_i = sum_{j<=i} phi(k_j) v_j^T,  z_i = sum_{j<=i} phi(k_j)
// with phi(x) = [exp(W x + b), exp(-(W x + b))] (section 3.4, Choices 1 and 3).
//
// How: the sequence of one (batch, head) is cut into segments, each segment
// into chunks of C = 64 tokens.  Per chunk, with Sp, zp the state before it:
//     y_c = (phiQ_c Sp + tril(phiQ_c phiK_c^T) V_c) / (phiQ_c zp + tril(phiQ_c phiK_c^T) 1)
//     Sp += phiK_c^T V_c,  zp += phiK_c^T 1
// which regroups the running sums of Eq. 2 exactly (only rounding differs).
// Three modes of one kernel template:
//   STATE   : segment aggregate dS = phiK^T V, dz = phiK^T 1 over the segment -> workspace
//   CAUSAL  : the chunk recurrence above, starting from the segment's prefix state
//   READOUT : y = phiQ S / phiQ z against a fixed total state (bidirectional mode)
// A separate scan kernel turns segment aggregates into exclusive prefixes.
//
// Work split inside a workgroup of NW waves (one wave per SIMD):
//   feature map : wave w computes directions [16 LB w, 16 LB (w+1)) for all 64 tokens
//                 (u^T = W x^T on MFMA, W rows held in registers), exp epilogue -> LDS
//   scores      : wave w computes query blocks [IBW w, IBW (w+1)) against key blocks <= them
//   read-out, intra-chunk product, state update: wave w owns value columns
//                 [16 VB w, 16 VB (w+1)) of S for every feature row, kept as fp32
//                 accumulators in registers for the whole segment
//   normaliser z: rows of z are split across waves; partial denominators meet in LDS.
#include "hh_common.h"
#include "hh_kernels.h"

namespace hh {

template <int D>
struct WideCfg {
    static constexpr int C = 64;                      // tokens per chunk
    static constexpr int NW = D == 128 ? 8 : (D == 64 ? 4 : D / 16);  // waves per workgroup
    static constexpr int NT = NW * 64;
    static constexpr int DP = 2 * D;                  // feature dimension
    static constexpr int FB = DP / 16;                // 16-row feature blocks
    static constexpr int KSF = DP / 32;               // 32-wide K steps over features
    static constexpr int KSD = (D + 31) / 32;         // K steps over the head dim (D = 16: half-filled)
    // feature map: NTH token groups x NDQ direction groups
    static constexpr int NTH = NW == 8 ? 2 : 1;
    static constexpr int NDQ = NW / NTH;
    static constexpr int DPW = D / NDQ;               // directions per wave
    static constexpr int LB = DPW / 16;               // direction blocks per wave
    static constexpr int IBT = 4 / NTH;               // token blocks per wave in the feature map
    // state: NF feature parts x NN value-column parts
    static constexpr int NF = NW == 8 ? 2 : 1;
    static constexpr int NN = NW / NF;
    static constexpr int VB = D / 16 / NN;            // value-column blocks per wave
    static constexpr int FBW = FB / NF;               // feature blocks per wave
    static constexpr int KSW = FBW / 2;               // read-out K steps per wave
    static constexpr int ZB = FB / NW;                // z-row blocks per wave
    static constexpr int IBF = 4 / NF;                // output row blocks finalised per wave
    static constexpr int NJ = NW == 8 ? 2 : 1;        // intra-chunk row-sum slots
    static constexpr int RQ = DP + 8;                 // row stride of [C][DP] tiles (bf16)
    static constexpr int RC = C + 8;                  // row stride of [*][C] tiles (bf16)
    static constexpr int XS = D + 4;                  // row stride of the fp32 exchange tile
    static constexpr int OFF_PQ = 0;
    static constexpr int OFF_PK = OFF_PQ + C * RQ * 2;     // also the exchange tile (NF = 2)
    static constexpr int OFF_PKT = OFF_PK + C * RQ * 2;
    static constexpr int OFF_VT = OFF_PKT + DP * RC * 2;
    static constexpr int OFF_A = OFF_VT + D * RC * 2;
    static constexpr int OFF_DEN = OFF_A + C * RC * 2;
    static constexpr int LDS_BYTES = OFF_DEN + (NW + NJ) * C * 4;
    static constexpr int MIN_WG_PER_CU = NW == 8 ? 1 : 2;
    static_assert(ZB == 2, "each wave owns one K step of z rows");
    static_assert(VB >= 1 && LB >= 1 && FBW % 2 == 0, "bad wave split");
    static_assert(NF == 1 || C * XS * 4 <= C * RQ * 2, "exchange tile must fit in the phiK tile");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
};

enum { WM_STATE = 0, WM_CAUSAL = 1, WM_READOUT = 2 };

// Position of feature f in a row-major feature tile.  With PERM, each 32-feature group is
// stored in the K order of two stacked accumulator blocks (lane group g reads features
// {4g..4g+3, 16+4g..16+4g+3} as one 16-byte run), so the read-out operand that pairs with
// the carried state is one 16-byte LDS read.  The scores read both tiles in the same
// (physical) order, which is a consistent permutation of their contraction index.
template <bool PERM>
__device__ __forceinline__ int feat_pos(int fbase4) {  // fbase4: first of 4 consecutive features, fbase4 % 4 == 0
    if (!PERM) return fbase4;
    const int fl = fbase4 & 31;
    return (fbase4 & ~31) + 8 * ((fl & 15) >> 2) + ((fl & 16) ? 4 : 0);
}

__device__ __forceinline__ uint32_t pack2(__bf16 lo, __bf16 hi) {
    bf16x2 v;
    v[0] = lo;
    v[1] = hi;
    return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ __bf16 lo16(uint32_t u) { return __builtin_bit_cast(bf16x2, u)[0]; }
__device__ __forceinline__ __bf16 hi16(uint32_t u) { return __builtin_bit_cast(bf16x2, u)[1]; }
// Exchange a 32-bit value with the neighbouring lane (lane ^ 1), a DPP quad permutation.
__device__ __forceinline__ uint32_t swap_adjacent(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);
}

// Write 4 features (rows f0 .. f0+3) of token i into a transposed tile [f][token] as 32-bit
// pairs of tokens: even lanes write rows f0, f0+1 for tokens (i, i+1), odd lanes rows f0+2,
// f0+3 for tokens (i-1, i), after swapping halves with the neighbouring lane.
template <int RC>
__device__ __forceinline__ void store_transposed_pairs(bf16_t *sT, int f0, int i, bool odd, const bf16x4 &v) {
    const uint32_t send = odd ? pack2(v[0], v[1]) : pack2(v[2], v[3]);
    const uint32_t recv = swap_adjacent(send);
    const int ie = i & ~1;
#pragma unroll
    for (int k = 0; k < 2; k++) {
        const __bf16 own = odd ? v[2 + k] : v[k];
        const __bf16 oth = k == 0 ? lo16(recv) : hi16(recv);
        const uint32_t word = odd ? pack2(oth, own) : pack2(own, oth);
        const int row = f0 + (odd ? 2 : 0) + k;
        *reinterpret_cast<uint32_t *>(sT + row * RC + ie) = word;
    }
}

// Feature map of one chunk for this wave's directions and token blocks, written to LDS.
//   ROWMAJOR : phi[i][pos(f)] (features contiguous), for the scores and the read-out
//   TRANS    : phi^T[f][i] (tokens contiguous), for the state update
template <int D, bool IS_KEY, bool FULL, bool ROWMAJOR, bool PERM, bool TRANS>
__device__ __forceinline__ void phi_chunk(const bf16_t *__restrict__ x, int t0, int valid,
                                          const bf16x8 (&wA)[WideCfg<D>::LB][WideCfg<D>::KSD],
                                          const float (&bl2)[WideCfg<D>::LB][4], int th, int dq, int g, int r16,
                                          bf16_t *sRow, bf16_t *sT) {
    using K = WideCfg<D>;
    f32x4 acc[K::LB][K::IBT];
#pragma unroll
    for (int ibl = 0; ibl < K::IBT; ibl++) {
        const int i = 16 * (th * K::IBT + ibl) + r16;
        bf16x8 xb[K::KSD];
#pragma unroll
        for (int ks = 0; ks < K::KSD; ks++) {
            const int m0 = 32 * ks + 8 * g;
            xb[ks] = ((FULL || i < valid) && m0 < D) ? load8(x + (size_t)(t0 + i) * D + m0) : zero_bf16x8();
        }
#pragma unroll
        for (int mb = 0; mb < K::LB; mb++) {
            f32x4 a = zero4();
#pragma unroll
            for (int ks = 0; ks < K::KSD; ks++) a = mfma_bf16(wA[mb][ks], xb[ks], a);
            acc[mb][ibl] = a;
        }
    }
    const bool odd = (r16 & 1) != 0;
#pragma unroll
    for (int mb = 0; mb < K::LB; mb++) {
        const int fb4 = dq * K::DPW + 16 * mb + 4 * g;  // this lane's 4 directions
#pragma unroll
        for (int ibl = 0; ibl < K::IBT; ibl++) {
            const int i = 16 * (th * K::IBT + ibl) + r16;
            f32x4 ep, en;
#pragma unroll
            for (int r = 0; r < 4; r++) {
                const float u = acc[mb][ibl][r] * kLog2e + bl2[mb][r];
                ep[r] = exp2_fast(u);
                en[r] = exp2_fast(-u);
            }
            if (IS_KEY && !FULL && i >= valid) {  // keys past the end contribute nothing
                ep = zero4();
                en = zero4();
            }
            const bf16x4 bp = to_bf16x4(ep), bn = to_bf16x4(en);
            if (ROWMAJOR) {
                store4(sRow + i * K::RQ + feat_pos<PERM>(fb4), bp);
                store4(sRow + i * K::RQ + feat_pos<PERM>(D + fb4), bn);
            }
            if (TRANS) {
                store_transposed_pairs<K::RC>(sT, fb4, i, odd, bp);
                store_transposed_pairs<K::RC>(sT, D + fb4, i, odd, bn);
            }
        }
    }
}

// Directions of direction group dq as MFMA A operands: row l = dq DPW + 16 mb + r16, K = input
// dim; bias pre-multiplied by log2(e) for the accumulator rows l = dq DPW + 16 mb + 4 g + r.
template <int D>
__device__ __forceinline__ void load_directions(const bf16_t *__restrict__ W, const bf16_t *__restrict__ b, int h,
                                                int dq, int g, int r16,
                                                bf16x8 (&wA)[WideCfg<D>::LB][WideCfg<D>::KSD],
                                                float (&bl2)[WideCfg<D>::LB][4]) {
    using K = WideCfg<D>;
    const bf16_t *Wh = W + (size_t)h * D * D;
#pragma unroll
    for (int mb = 0; mb < K::LB; mb++) {
        const int l = dq * K::DPW + 16 * mb + r16;
#pragma unroll
        for (int ks = 0; ks < K::KSD; ks++) {
            const int m0 = 32 * ks + 8 * g;
            wA[mb][ks] = (m0 < D) ? load8(Wh + (size_t)l * D + m0) : zero_bf16x8();
        }
#pragma unroll
        for (int r = 0; r < 4; r++) {
            const int lb = dq * K::DPW + 16 * mb + 4 * g + r;
            bl2[mb][r] = b ? bf16_bits_to_float(b[(size_t)h * D + lb]) * kLog2e : 0.0f;
        }
    }
}

// V chunk [C][D] -> LDS as V^T [D][C] (tokens contiguous); rows past the end are zero.
// Lanes 2p and 2p+1 load the same 8 columns of tokens j and j+1 (16 bytes each), swap four
// columns and write 32-bit token pairs.
template <int D, bool FULL>
__device__ __forceinline__ void v_chunk_to_lds(const bf16_t *__restrict__ v, int t0, int valid, int tid,
                                               bf16_t *sVT) {
    using K = WideCfg<D>;
    constexpr int NC = D / 8;
    constexpr int PIECES = K::C * NC;
    static_assert(PIECES % K::NT == 0, "every lane takes part in each pass");
#pragma unroll
    for (int it = 0; it < PIECES / K::NT; it++) {
        const int t = tid + it * K::NT;
        const int pr = t >> 1;
        const bool odd = (t & 1) != 0;
        const int nc = pr % NC, j = 2 * (pr / NC) + (odd ? 1 : 0);
        const bf16x8 val = (FULL || j < valid) ? load8(v + (size_t)(t0 + j) * D + 8 * nc) : zero_bf16x8();
        // even lanes keep columns 0..3 and send 4..7; odd lanes keep 4..7 and send 0..3
        const uint32_t s0 = odd ? pack2(val[0], val[1]) : pack2(val[4], val[5]);
        const uint32_t s1 = odd ? pack2(val[2], val[3]) : pack2(val[6], val[7]);
        const uint32_t r0 = swap_adjacent(s0), r1 = swap_adjacent(s1);
        const __bf16 oth[4] = {lo16(r0), hi16(r0), lo16(r1), hi16(r1)};
        const int je = j & ~1;
#pragma unroll
        for (int c = 0; c < 4; c++) {
            const __bf16 own = odd ? val[4 + c] : val[c];
            const uint32_t word = odd ? pack2(oth[c], own) : pack2(own, oth[c]);
            *reinterpret_cast<uint32_t *>(sVT + (8 * nc + (odd ? 4 : 0) + c) * K::RC + je) = word;
        }
    }
}

// Query blocks and key-block range of the intra-chunk scores handled by wave w, and the
// row-sum slot it writes.  Every (query block, key block <= it) pair is covered once.
template <int NW>
__device__ __forceinline__ void score_task(int w, int qq, int &ib, int &jlo, int &jhi, int &slot) {
    if (NW == 8) {
        ib = w & 3;
        jlo = w < 4 ? 0 : 2;
        jhi = w < 4 ? (ib < 1 ? ib : 1) : ib;
        slot = w >> 2;
    } else {
        ib = w * (4 / NW) + qq;
        jlo = 0;
        jhi = ib;
        slot = 0;
    }
}

template <int D, int MODE, bool FULL>
__device__ __forceinline__ void chunk_step(const WideParams &p, size_t base, int t0, int valid, unsigned char *smem,
                                           const bf16x8 (&wA)[WideCfg<D>::LB][WideCfg<D>::KSD],
                                           const float (&bl2)[WideCfg<D>::LB][4],
                                           f32x4 (&sacc)[WideCfg<D>::FBW][WideCfg<D>::VB],
                                           f32x4 (&zacc)[WideCfg<D>::ZB], int tid) {
    using K = WideCfg<D>;
    bf16_t *sPQ = reinterpret_cast<bf16_t *>(smem + K::OFF_PQ);
    bf16_t *sPK = reinterpret_cast<bf16_t *>(smem + K::OFF_PK);
    bf16_t *sPKT = reinterpret_cast<bf16_t *>(smem + K::OFF_PKT);
    bf16_t *sVT = reinterpret_cast<bf16_t *>(smem + K::OFF_VT);
    bf16_t *sA = reinterpret_cast<bf16_t *>(smem + K::OFF_A);
    float *sDen = reinterpret_cast<float *>(smem + K::OFF_DEN);
    float *sX = reinterpret_cast<float *>(smem + K::OFF_PK);
    const int w = tid >> 6, lane = tid & 63, g = lane >> 4, r16 = lane & 15;
    const int th = w / K::NDQ, dq = w % K::NDQ;  // feature-map role
    const int fa = w / K::NN, nq = w % K::NN;     // state role: feature part, value part

    // ---- phase 1: feature maps and V^T into LDS
    if (MODE == WM_CAUSAL)
        phi_chunk<D, true, FULL, true, true, true>(p.k + base, t0, valid, wA, bl2, th, dq, g, r16, sPK, sPKT);
    if (MODE == WM_STATE)
        phi_chunk<D, true, FULL, false, true, true>(p.k + base, t0, valid, wA, bl2, th, dq, g, r16, nullptr, sPKT);
    if (MODE != WM_STATE)
        phi_chunk<D, false, FULL, true, true, false>(p.q + base, t0, valid, wA, bl2, th, dq, g, r16, sPQ, nullptr);
    if (MODE != WM_READOUT) v_chunk_to_lds<D, FULL>(p.v + base, t0, valid, tid, sVT);
    __syncthreads();

    f32x4 num[4][K::VB];
    if (MODE != WM_STATE) {
        // ---- phase 2: intra-chunk scores, read-out against the carried state, denominators
        if (MODE == WM_CAUSAL) {
#pragma unroll
            for (int qq = 0; qq < (K::NW >= 4 ? 1 : 4 / K::NW); qq++) {
                int ib, jlo, jhi, slot;
                score_task<K::NW>(w, qq, ib, jlo, jhi, slot);
                constexpr int MAXJ = K::NW == 8 ? 2 : 4;
                f32x4 a[MAXJ];
#pragma unroll
                for (int jj = 0; jj < MAXJ; jj++) a[jj] = zero4();
#pragma unroll
                for (int ks = 0; ks < K::KSF; ks++) {
                    const bf16x8 qb = load8(sPQ + (16 * ib + r16) * K::RQ + 32 * ks + 8 * g);
#pragma unroll
                    for (int jj = 0; jj < MAXJ; jj++)
                        if (jlo + jj <= jhi)
                            a[jj] = mfma_bf16(load8(sPK + (16 * (jlo + jj) + r16) * K::RQ + 32 * ks + 8 * g), qb, a[jj]);
                }
                float rs = 0.0f;
#pragma unroll
                for (int jj = 0; jj < MAXJ; jj++) {
                    const int jb = jlo + jj;
                    if (jb > jhi) continue;
                    // a = A^T[j][i]: lane holds i = 16 ib + r16, j = 16 jb + 4 g + r; keep j <= i
                    f32x4 av = a[jj];
                    if (jb == ib) {
#pragma unroll
                        for (int r = 0; r < 4; r++)
                            if (4 * g + r > r16) av[r] = 0.0f;
                    }
                    const bf16x4 ab = to_bf16x4(av);
                    rs += ((float)ab[0] + (float)ab[1]) + ((float)ab[2] + (float)ab[3]);
                    store4(sA + (16 * ib + r16) * K::RC + 16 * jb + 4 * g, ab);
                }
                if (jlo == 0 && (ib & 1) == 0) {  // the K step covering block ib also covers block ib + 1
                    bf16x4 zz;
                    zz[0] = zz[1] = zz[2] = zz[3] = (__bf16)0.0f;
                    store4(sA + (16 * ib + r16) * K::RC + 16 * (ib + 1) + 4 * g, zz);
                }
                rs += __shfl_xor(rs, 16);
                rs += __shfl_xor(rs, 32);
                if (g == 0) sDen[(K::NW + slot) * K::C + 16 * ib + r16] = rs;
            }
        }
#pragma unroll
        for (int ib = 0; ib < 4; ib++)
#pragma unroll
            for (int vb = 0; vb < K::VB; vb++) num[ib][vb] = zero4();
#pragma unroll
        for (int kk = 0; kk < K::KSW; kk++) {
            const int ks = fa * K::KSW + kk;
            bf16x8 sb[K::VB];
#pragma unroll
            for (int vb = 0; vb < K::VB; vb++) sb[vb] = acc_pair_to_operand(sacc[2 * kk][vb], sacc[2 * kk + 1][vb]);
#pragma unroll
            for (int ib = 0; ib < 4; ib++) {
                const bf16x8 a = load8(sPQ + (16 * ib + r16) * K::RQ + 32 * ks + 8 * g);
#pragma unroll
                for (int vb = 0; vb < K::VB; vb++) num[ib][vb] = mfma_bf16(a, sb[vb], num[ib][vb]);
            }
        }
        {  // partial denominators over this wave's z rows (K step w of the features)
            const bf16x8 zb = acc_pair_to_operand(zacc[0], zacc[1]);
#pragma unroll
            for (int ib = 0; ib < 4; ib++) {
                const f32x4 dacc = mfma_bf16(load8(sPQ + (16 * ib + r16) * K::RQ + 32 * w + 8 * g), zb, zero4());
                if (r16 == 0) *reinterpret_cast<f32x4 *>(sDen + w * K::C + 16 * ib + 4 * g) = dacc;
            }
        }
        if (K::NF == 2) {
            __syncthreads();  // every wave is done with the phiK tile: reuse it for the exchange
#pragma unroll
            for (int ib = 0; ib < 4; ib++) {
                if (ib / K::IBF == fa) continue;
#pragma unroll
                for (int vb = 0; vb < K::VB; vb++) {
                    const int n = 16 * (nq * K::VB + vb) + r16;
#pragma unroll
                    for (int r = 0; r < 4; r++) sX[(16 * ib + 4 * g + r) * K::XS + n] = num[ib][vb][r];
                }
            }
        }
    }
    __syncthreads();

    // ---- phase 3: exchange, intra-chunk product, output, state update
    bf16x8 vop[2][K::VB];
    if (MODE != WM_READOUT) {
#pragma unroll
        for (int ks = 0; ks < 2; ks++)
#pragma unroll
            for (int vb = 0; vb < K::VB; vb++)
                vop[ks][vb] = load8(sVT + (16 * (nq * K::VB + vb) + r16) * K::RC + 32 * ks + 8 * g);
    }
    if (MODE != WM_STATE) {
        bf16_t *yb = p.y + base + (size_t)t0 * D;
#pragma unroll
        for (int ib = 0; ib < 4; ib++) {
            if (ib / K::IBF != fa) continue;  // rows finalised by the other feature part
            const int i0 = 16 * ib + 4 * g;
            if (K::NF == 2) {
#pragma unroll
                for (int vb = 0; vb < K::VB; vb++) {
                    const int n = 16 * (nq * K::VB + vb) + r16;
#pragma unroll
                    for (int r = 0; r < 4; r++) num[ib][vb][r] += sX[(i0 + r) * K::XS + n];
                }
            }
            if (MODE == WM_CAUSAL) {
#pragma unroll
                for (int ks = 0; ks <= ib / 2; ks++) {
                    const bf16x8 a = load8(sA + (16 * ib + r16) * K::RC + 32 * ks + 8 * g);
#pragma unroll
                    for (int vb = 0; vb < K::VB; vb++) num[ib][vb] = mfma_bf16(a, vop[ks][vb], num[ib][vb]);
                }
            }
            f32x4 den = zero4();
#pragma unroll
            for (int pw = 0; pw < K::NW + (MODE == WM_CAUSAL ? K::NJ : 0); pw++)
                den += *reinterpret_cast<const f32x4 *>(sDen + pw * K::C + i0);
            f32x4 rden;
#pragma unroll
            for (int r = 0; r < 4; r++) rden[r] = __builtin_amdgcn_rcpf(den[r]);
#pragma unroll
            for (int vb = 0; vb < K::VB; vb++) {
                const int n = 16 * (nq * K::VB + vb) + r16;
#pragma unroll
                for (int r = 0; r < 4; r++)
                    if (FULL || i0 + r < valid) yb[(size_t)(i0 + r) * D + n] = float_to_bf16_bits(num[ib][vb][r] * rden[r]);
            }
        }
    }
    if (MODE != WM_READOUT) {
        const bf16x8 ones = ones_bf16x8();
#pragma unroll
        for (int fb = 0; fb < K::FBW; fb++)
#pragma unroll
            for (int ks = 0; ks < 2; ks++) {
                const bf16x8 a = load8(sPKT + (16 * (fa * K::FBW + fb) + r16) * K::RC + 32 * ks + 8 * g);
#pragma unroll
                for (int vb = 0; vb < K::VB; vb++) sacc[fb][vb] = mfma_bf16(a, vop[ks][vb], sacc[fb][vb]);
            }
#pragma unroll
        for (int zb = 0; zb < K::ZB; zb++)
#pragma unroll
            for (int ks = 0; ks < 2; ks++) {
                const bf16x8 a = load8(sPKT + (16 * (w * K::ZB + zb) + r16) * K::RC + 32 * ks + 8 * g);
                zacc[zb] = mfma_bf16(a, ones, zacc[zb]);
            }
    }
    __syncthreads();
}

template <int D, int MODE>
__global__ __launch_bounds__(WideCfg<D>::NT, WideCfg<D>::MIN_WG_PER_CU) void wide_kernel(WideParams p) {
    using K = WideCfg<D>;
    __shared__ __attribute__((aligned(16))) unsigned char smem[K::LDS_BYTES];

    const int tid = threadIdx.x;
    const int w = tid >> 6, lane = tid & 63, g = lane >> 4, r16 = lane & 15;
    const int dq = w % K::NDQ;
    const int fa = w / K::NN, nq = w % K::NN;
    const int bh = blockIdx.x / p.nseg_grid;
    const int s = blockIdx.x % p.nseg_grid;
    const int h = bh % p.H;
    const int t_begin = s * p.seg_len;
    const int t_end = min(p.N, t_begin + p.seg_len);
    const size_t base = (size_t)bh * p.N * D;

    bf16x8 wA[K::LB][K::KSD];
    float bl2[K::LB][4];
    load_directions<D>(p.W, p.b, h, dq, g, r16, wA, bl2);

    // State: S[f][n] for feature blocks fa*FBW .. and this wave's value columns; z rows of
    // feature blocks w*ZB .. (every column of the z accumulator holds the same value).
    f32x4 sacc[K::FBW][K::VB];
    f32x4 zacc[K::ZB];
    {
        const float *Si = nullptr, *zi = nullptr;
        if (MODE != WM_STATE && p.S_in) {
            const size_t slot = (size_t)bh * p.in_bh_stride + (size_t)s * p.in_seg_stride;
            Si = p.S_in + slot * K::DP * D;
            zi = p.z_in + slot * K::DP;
        }
#pragma unroll
        for (int fb = 0; fb < K::FBW; fb++)
#pragma unroll
            for (int vb = 0; vb < K::VB; vb++) {
                const int n = 16 * (nq * K::VB + vb) + r16;
#pragma unroll
                for (int r = 0; r < 4; r++)
                    sacc[fb][vb][r] = Si ? Si[(size_t)(16 * (fa * K::FBW + fb) + 4 * g + r) * D + n] : 0.0f;
            }
#pragma unroll
        for (int zb = 0; zb < K::ZB; zb++)
#pragma unroll
            for (int r = 0; r < 4; r++) zacc[zb][r] = zi ? zi[16 * (w * K::ZB + zb) + 4 * g + r] : 0.0f;
    }

    int t0 = t_begin;
    for (; t0 + K::C <= t_end; t0 += K::C)
        chunk_step<D, MODE, true>(p, base, t0, K::C, smem, wA, bl2, sacc, zacc, tid);
    if (t0 < t_end) chunk_step<D, MODE, false>(p, base, t0, t_end - t0, smem, wA, bl2, sacc, zacc, tid);

    // ---- segment end: publish the aggregate (STATE) or the final state (CAUSAL, last segment)
    float *So = nullptr, *zo = nullptr;
    if (MODE == WM_STATE) {
        const size_t slot = (size_t)bh * p.ws_bh_stride + s;
        So = p.S_ws + slot * K::DP * D;
        zo = p.z_ws + slot * K::DP;
    } else if (MODE == WM_CAUSAL && p.S_out && s == p.nseg_grid - 1) {
        So = p.S_out + (size_t)bh * K::DP * D;
        zo = p.z_out + (size_t)bh * K::DP;
    }
    if (So) {
#pragma unroll
        for (int fb = 0; fb < K::FBW; fb++)
#pragma unroll
            for (int vb = 0; vb < K::VB; vb++) {
                const int n = 16 * (nq * K::VB + vb) + r16;
#pragma unroll
                for (int r = 0; r < 4; r++) So[(size_t)(16 * (fa * K::FBW + fb) + 4 * g + r) * D + n] = sacc[fb][vb][r];
            }
        if (r16 == 0) {
#pragma unroll
            for (int zb = 0; zb < K::ZB; zb++)
#pragma unroll
                for (int r = 0; r < 4; r++) zo[16 * (w * K::ZB + zb) + 4 * g + r] = zacc[zb][r];
        }
    }
}

// Stand-alone feature map: each workgroup maps `cpw` chunks of 64 tokens of one head and
// writes phi [token][2d] through an LDS tile so that global stores are full 16-byte rows.
template <int D>
__global__ __launch_bounds__(WideCfg<D>::NT, WideCfg<D>::MIN_WG_PER_CU) void fm_hedgehog_kernel(const bf16_t *__restrict__ x,
                                                                        const bf16_t *__restrict__ W,
                                                                        const bf16_t *__restrict__ b,
                                                                        bf16_t *__restrict__ phi, int H, int N,
                                                                        int cpw, int wg_per_bh) {
    using K = WideCfg<D>;
    __shared__ __attribute__((aligned(16))) bf16_t sPhi[K::C * K::RQ];
    const int tid = threadIdx.x;
    const int w = tid >> 6, lane = tid & 63, g = lane >> 4, r16 = lane & 15;
    const int th = w / K::NDQ, dq = w % K::NDQ;
    const int bh = blockIdx.x / wg_per_bh, part = blockIdx.x % wg_per_bh;
    const int h = bh % H;
    bf16x8 wA[K::LB][K::KSD];
    float bl2[K::LB][4];
    load_directions<D>(W, b, h, dq, g, r16, wA, bl2);
    const bf16_t *xh = x + (size_t)bh * N * D;
    bf16_t *ph = phi + (size_t)bh * N * K::DP;
    for (int c = 0; c < cpw; c++) {
        const int t0 = (part * cpw + c) * K::C;
        if (t0 >= N) break;
        const int valid = min(K::C, N - t0);
        if (valid == K::C)
            phi_chunk<D, false, true, true, false, false>(xh, t0, valid, wA, bl2, th, dq, g, r16, sPhi, nullptr);
        else
            phi_chunk<D, false, false, true, false, false>(xh, t0, valid, wA, bl2, th, dq, g, r16, sPhi, nullptr);
        __syncthreads();
        constexpr int P8 = K::DP / 8;
        for (int pi = tid; pi < K::C * P8; pi += K::NT) {
            const int i = pi / P8, c8 = pi % P8;
            if (i < valid) store8(ph + (size_t)(t0 + i) * K::DP + 8 * c8, load8(sPhi + i * K::RQ + 8 * c8));
        }
        __syncthreads();
    }
}

template <int D>
static hipError_t launch_fm_d(const bf16_t *x, const bf16_t *W, const bf16_t *b, bf16_t *phi, int BH, int H, int N,
                              hipStream_t st) {
    using K = WideCfg<D>;
    const long nch = (N + K::C - 1) / K::C;
    // enough workgroups to fill the chip, several chunks each to amortise loading W
    long cpw = ((long)BH * nch) / 1024;
    if (cpw < 1) cpw = 1;
    if (cpw > 8) cpw = 8;
    const long wpb = (nch + cpw - 1) / cpw;
    hipLaunchKernelGGL((fm_hedgehog_kernel<D>), dim3((unsigned)(BH * wpb)), dim3(K::NT), 0, st, x, W, b, phi, H, N,
                       (int)cpw, (int)wpb);
    return hipGetLastError();
}

hipError_t launch_featuremap_hedgehog_bf16(int d, const bf16_t *x, const bf16_t *W, const bf16_t *b, bf16_t *phi,
                                           int BH, int H, int N, hipStream_t st) {
    switch (d) {
    case 16: return launch_fm_d<16>(x, W, b, phi, BH, H, N, st);
    case 32: return launch_fm_d<32>(x, W, b, phi, BH, H, N, st);
    case 64: return launch_fm_d<64>(x, W, b, phi, BH, H, N, st);
    case 128: return launch_fm_d<128>(x, W, b, phi, BH, H, N, st);
    default: return hipErrorInvalidValue;
    }
}

template <int D>
static hipError_t launch_wide_d(int mode, const WideParams &p, int grid, hipStream_t st) {
    using K = WideCfg<D>;
    switch (mode) {
    case WM_STATE:
        hipLaunchKernelGGL((wide_kernel<D, WM_STATE>), dim3(grid), dim3(K::NT), 0, st, p);
        break;
    case WM_CAUSAL:
        hipLaunchKernelGGL((wide_kernel<D, WM_CAUSAL>), dim3(grid), dim3(K::NT), 0, st, p);
        break;
    default:
        hipLaunchKernelGGL((wide_kernel<D, WM_READOUT>), dim3(grid), dim3(K::NT), 0, st, p);
        break;
    }
    return hipGetLastError();
}

hipError_t launch_wide(int d, int mode, const WideParams &p, int grid, hipStream_t st) {
    switch (d) {
    case 16: return launch_wide_d<16>(mode, p, grid, st);
    case 32: return launch_wide_d<32>(mode, p, grid, st);
    case 64: return launch_wide_d<64>(mode, p, grid, st);
    case 128: return launch_wide_d<128>(mode, p, grid, st);
    default: return hipErrorInvalidValue;
    }
}

int wide_wgs_per_cu(int d) {
    int lds = 0;
    switch (d) {
    case 16: lds = WideCfg<16>::LDS_BYTES; break;
    case 32: lds = WideCfg<32>::LDS_BYTES; break;
    case 64: lds = WideCfg<64>::LDS_BYTES; break;
    case 128: lds = WideCfg<128>::LDS_BYTES; break;
    default: return 1;
    }
    int n = (160 * 1024) / lds;
    if (d == 128) n = 1;  // 8 waves per workgroup already fill the CU
    return n < 1 ? 1 : (n > 4 ? 4 : n);
}

}  // namespace hh
