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
    static constexpr int C = 64;                     // tokens per chunk
    static constexpr int NW = D >= 64 ? 4 : D / 16;  // waves per workgroup
    static constexpr int NT = NW * 64;
    static constexpr int DP = 2 * D;                 // feature dimension
    static constexpr int FB = DP / 16;               // 16-row feature blocks
    static constexpr int KSF = DP / 32;              // 32-wide K steps over features
    static constexpr int KSD = (D + 31) / 32;        // K steps over the head dim (D = 16: half-filled)
    static constexpr int VB = D / 16 / NW;           // value-column blocks per wave
    static constexpr int LB = VB;                    // direction blocks per wave
    static constexpr int ZB = FB / NW;               // z-row blocks per wave
    static constexpr int IBW = 4 / NW;               // query blocks per wave in the scores
    static constexpr int RQ = DP + 8;                // row stride of [C][DP] tiles (bf16)
    static constexpr int RC = C + 8;                 // row stride of [*][C] tiles (bf16)
    static constexpr int OFF_PQ = 0;
    static constexpr int OFF_PK = OFF_PQ + C * RQ * 2;
    static constexpr int OFF_PKT = OFF_PK + C * RQ * 2;
    static constexpr int OFF_VT = OFF_PKT + DP * RC * 2;
    static constexpr int OFF_A = OFF_VT + D * RC * 2;
    static constexpr int OFF_DEN = OFF_A + C * RC * 2;
    static constexpr int LDS_BYTES = OFF_DEN + (NW + 1) * C * 4;
    static_assert(ZB % 2 == 0, "z rows per wave must cover whole K steps");
    static_assert(VB >= 1 && LB >= 1, "bad wave split");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
};

enum { WM_STATE = 0, WM_CAUSAL = 1, WM_READOUT = 2 };

// Feature map of one chunk for this wave's directions, written to LDS.
//   ROWMAJOR : phi[i][f] (f contiguous), for the scores and the read-out
//   TRANS    : phi^T[f][i] (tokens contiguous), for the state update
template <int D, bool IS_KEY, bool ROWMAJOR, bool TRANS>
__device__ __forceinline__ void phi_chunk(const bf16_t *__restrict__ x, int t0, int valid,
                                          const bf16x8 (&wA)[WideCfg<D>::LB][WideCfg<D>::KSD],
                                          const float (&bl2)[WideCfg<D>::LB][4], int w, int g, int r16,
                                          bf16_t *sRow, bf16_t *sT) {
    using K = WideCfg<D>;
    f32x4 acc[K::LB][4];
#pragma unroll
    for (int ib = 0; ib < 4; ib++) {
        const int i = 16 * ib + r16;
        bf16x8 xb[K::KSD];
#pragma unroll
        for (int ks = 0; ks < K::KSD; ks++) {
            const int m0 = 32 * ks + 8 * g;
            xb[ks] = (i < valid && m0 < D) ? load8(x + (size_t)(t0 + i) * D + m0) : zero_bf16x8();
        }
#pragma unroll
        for (int mb = 0; mb < K::LB; mb++) {
            f32x4 a = zero4();
#pragma unroll
            for (int ks = 0; ks < K::KSD; ks++) a = mfma_bf16(wA[mb][ks], xb[ks], a);
            acc[mb][ib] = a;
        }
    }
    // acc[mb][ib]: lane holds u for token i = 16 ib + r16 and directions l0 + r
#pragma unroll
    for (int mb = 0; mb < K::LB; mb++) {
        const int l0 = 16 * (w * K::LB + mb) + 4 * g;
#pragma unroll
        for (int ib = 0; ib < 4; ib++) {
            const int i = 16 * ib + r16;
            f32x4 ep, en;
#pragma unroll
            for (int r = 0; r < 4; r++) {
                const float u = acc[mb][ib][r] * kLog2e + bl2[mb][r];
                ep[r] = exp2_fast(u);
                en[r] = exp2_fast(-u);
            }
            if (IS_KEY && i >= valid) {  // keys past the end contribute nothing
                ep = zero4();
                en = zero4();
            }
            const bf16x4 bp = to_bf16x4(ep), bn = to_bf16x4(en);
            if (ROWMAJOR) {
                store4(sRow + i * K::RQ + l0, bp);
                store4(sRow + i * K::RQ + D + l0, bn);
            }
            if (TRANS) {
#pragma unroll
                for (int r = 0; r < 4; r++) {
                    reinterpret_cast<__bf16 *>(sT)[(l0 + r) * K::RC + i] = bp[r];
                    reinterpret_cast<__bf16 *>(sT)[(D + l0 + r) * K::RC + i] = bn[r];
                }
            }
        }
    }
}

// Directions of wave w as MFMA A operands: row l = 16 (w LB + mb) + r16, K = input dim;
// bias pre-multiplied by log2(e) for the rows l = 16 (w LB + mb) + 4 g + r of the accumulator.
template <int D>
__device__ __forceinline__ void load_directions(const bf16_t *__restrict__ W, const bf16_t *__restrict__ b, int h,
                                                int w, int g, int r16,
                                                bf16x8 (&wA)[WideCfg<D>::LB][WideCfg<D>::KSD],
                                                float (&bl2)[WideCfg<D>::LB][4]) {
    using K = WideCfg<D>;
    const bf16_t *Wh = W + (size_t)h * D * D;
#pragma unroll
    for (int mb = 0; mb < K::LB; mb++) {
        const int l = 16 * (w * K::LB + mb) + r16;
#pragma unroll
        for (int ks = 0; ks < K::KSD; ks++) {
            const int m0 = 32 * ks + 8 * g;
            wA[mb][ks] = (m0 < D) ? load8(Wh + (size_t)l * D + m0) : zero_bf16x8();
        }
#pragma unroll
        for (int r = 0; r < 4; r++) {
            const int lb = 16 * (w * K::LB + mb) + 4 * g + r;
            bl2[mb][r] = b ? bf16_bits_to_float(b[(size_t)h * D + lb]) * kLog2e : 0.0f;
        }
    }
}

// V chunk [C][D] -> LDS as V^T [D][C] (tokens contiguous); rows past the end are zero.
template <int D>
__device__ __forceinline__ void v_chunk_to_lds(const bf16_t *__restrict__ v, int t0, int valid, int tid,
                                               bf16_t *sVT) {
    using K = WideCfg<D>;
    constexpr int NC = D / 8;
    for (int t = tid; t < (K::C / 4) * NC; t += K::NT) {
        const int jq = t / NC, nc = t % NC;
        bf16x8 rows[4];
#pragma unroll
        for (int jj = 0; jj < 4; jj++) {
            const int j = 4 * jq + jj;
            rows[jj] = (j < valid) ? load8(v + (size_t)(t0 + j) * D + 8 * nc) : zero_bf16x8();
        }
#pragma unroll
        for (int c = 0; c < 8; c++) {
            bf16x4 col;
            col[0] = rows[0][c];
            col[1] = rows[1][c];
            col[2] = rows[2][c];
            col[3] = rows[3][c];
            *reinterpret_cast<bf16x4 *>(sVT + (8 * nc + c) * K::RC + 4 * jq) = col;
        }
    }
}

template <int D, int MODE>
__global__ __launch_bounds__(WideCfg<D>::NT, 1) void wide_kernel(WideParams p) {
    using K = WideCfg<D>;
    __shared__ __attribute__((aligned(16))) unsigned char smem[K::LDS_BYTES];
    bf16_t *sPQ = reinterpret_cast<bf16_t *>(smem + K::OFF_PQ);
    bf16_t *sPK = reinterpret_cast<bf16_t *>(smem + K::OFF_PK);
    bf16_t *sPKT = reinterpret_cast<bf16_t *>(smem + K::OFF_PKT);
    bf16_t *sVT = reinterpret_cast<bf16_t *>(smem + K::OFF_VT);
    bf16_t *sA = reinterpret_cast<bf16_t *>(smem + K::OFF_A);
    float *sDen = reinterpret_cast<float *>(smem + K::OFF_DEN);

    const int tid = threadIdx.x;
    const int w = tid >> 6, lane = tid & 63, g = lane >> 4, r16 = lane & 15;
    const int bh = blockIdx.x / p.nseg_grid;
    const int s = blockIdx.x % p.nseg_grid;
    const int h = bh % p.H;
    const int t_begin = s * p.seg_len;
    const int t_end = min(p.N, t_begin + p.seg_len);
    const size_t base = (size_t)bh * p.N * D;

    bf16x8 wA[K::LB][K::KSD];
    float bl2[K::LB][4];
    load_directions<D>(p.W, p.b, h, w, g, r16, wA, bl2);

    // State: S[f][n] for this wave's value columns (all f), z[f] for this wave's z rows.
    f32x4 sacc[K::FB][K::VB];
    f32x4 zacc[K::ZB];
    {
        const float *Si = nullptr, *zi = nullptr;
        if (MODE != WM_STATE && p.S_in) {
            const size_t slot = (size_t)bh * p.in_bh_stride + (size_t)s * p.in_seg_stride;
            Si = p.S_in + slot * K::DP * D;
            zi = p.z_in + slot * K::DP;
        }
#pragma unroll
        for (int fb = 0; fb < K::FB; fb++)
#pragma unroll
            for (int vb = 0; vb < K::VB; vb++) {
                const int n = 16 * (w * K::VB + vb) + r16;
#pragma unroll
                for (int r = 0; r < 4; r++)
                    sacc[fb][vb][r] = Si ? Si[(size_t)(16 * fb + 4 * g + r) * D + n] : 0.0f;
            }
#pragma unroll
        for (int zb = 0; zb < K::ZB; zb++)
#pragma unroll
            for (int r = 0; r < 4; r++)
                zacc[zb][r] = zi ? zi[16 * (w * K::ZB + zb) + 4 * g + r] : 0.0f;
    }
    const bf16x8 ones = ones_bf16x8();

    for (int t0 = t_begin; t0 < t_end; t0 += K::C) {
        const int valid = min(K::C, t_end - t0);

        // ---- phase 1: feature maps and V^T into LDS
        if (MODE == WM_CAUSAL)
            phi_chunk<D, true, true, true>(p.k + base, t0, valid, wA, bl2, w, g, r16, sPK, sPKT);
        if (MODE == WM_STATE)
            phi_chunk<D, true, false, true>(p.k + base, t0, valid, wA, bl2, w, g, r16, sPK, sPKT);
        if (MODE != WM_STATE)
            phi_chunk<D, false, true, false>(p.q + base, t0, valid, wA, bl2, w, g, r16, sPQ, nullptr);
        if (MODE != WM_READOUT) v_chunk_to_lds<D>(p.v + base, t0, valid, tid, sVT);
        __syncthreads();

        f32x4 num[4][K::VB];
        // ---- phase 2: intra-chunk scores, read-out against the carried state, denominators
        if (MODE == WM_CAUSAL) {
#pragma unroll
            for (int qq = 0; qq < K::IBW; qq++) {
                const int ib = w * K::IBW + qq;
                bf16x8 qb[K::KSF];
#pragma unroll
                for (int ks = 0; ks < K::KSF; ks++) qb[ks] = load8(sPQ + (16 * ib + r16) * K::RQ + 32 * ks + 8 * g);
                float rs = 0.0f;
                for (int jb = 0; jb <= ib; jb++) {
                    f32x4 a = zero4();
#pragma unroll
                    for (int ks = 0; ks < K::KSF; ks++)
                        a = mfma_bf16(load8(sPK + (16 * jb + r16) * K::RQ + 32 * ks + 8 * g), qb[ks], a);
                    // a: A^T[j][i], lane holds i = 16 ib + r16, j = 16 jb + 4 g + r; keep j <= i
                    if (jb == ib) {
#pragma unroll
                        for (int r = 0; r < 4; r++)
                            if (4 * g + r > r16) a[r] = 0.0f;
                    }
                    const bf16x4 ab = to_bf16x4(a);
                    rs += (float)ab[0] + (float)ab[1] + (float)ab[2] + (float)ab[3];
                    store4(sA + (16 * ib + r16) * K::RC + 16 * jb + 4 * g, ab);
                }
                if ((ib & 1) == 0) {  // the K step covering block ib also covers block ib + 1
                    bf16x4 zz;
                    zz[0] = zz[1] = zz[2] = zz[3] = (__bf16)0.0f;
                    store4(sA + (16 * ib + r16) * K::RC + 16 * (ib + 1) + 4 * g, zz);
                }
                rs += __shfl_xor(rs, 16);
                rs += __shfl_xor(rs, 32);
                if (g == 0) sDen[K::NW * K::C + 16 * ib + r16] = rs;
            }
        }
        if (MODE != WM_STATE) {
#pragma unroll
            for (int ib = 0; ib < 4; ib++)
#pragma unroll
                for (int vb = 0; vb < K::VB; vb++) num[ib][vb] = zero4();
#pragma unroll
            for (int ks = 0; ks < K::KSF; ks++) {
                bf16x8 sb[K::VB];
#pragma unroll
                for (int vb = 0; vb < K::VB; vb++) sb[vb] = acc_pair_to_operand(sacc[2 * ks][vb], sacc[2 * ks + 1][vb]);
#pragma unroll
                for (int ib = 0; ib < 4; ib++) {
                    const bf16_t *rp = sPQ + (16 * ib + r16) * K::RQ + 32 * ks + 4 * g;
                    const bf16x8 a = cat(load4(rp), load4(rp + 16));
#pragma unroll
                    for (int vb = 0; vb < K::VB; vb++) num[ib][vb] = mfma_bf16(a, sb[vb], num[ib][vb]);
                }
            }
            // partial denominators over this wave's z rows
            f32x4 dacc[4];
#pragma unroll
            for (int ib = 0; ib < 4; ib++) dacc[ib] = zero4();
#pragma unroll
            for (int kz = 0; kz < K::ZB / 2; kz++) {
                const int ks = w * (K::ZB / 2) + kz;
                const bf16x8 zb = acc_pair_to_operand(zacc[2 * kz], zacc[2 * kz + 1]);
#pragma unroll
                for (int ib = 0; ib < 4; ib++) {
                    const bf16_t *rp = sPQ + (16 * ib + r16) * K::RQ + 32 * ks + 4 * g;
                    dacc[ib] = mfma_bf16(cat(load4(rp), load4(rp + 16)), zb, dacc[ib]);
                }
            }
            if (r16 == 0) {
#pragma unroll
                for (int ib = 0; ib < 4; ib++)
                    *reinterpret_cast<f32x4 *>(sDen + w * K::C + 16 * ib + 4 * g) = dacc[ib];
            }
        }
        __syncthreads();

        // ---- phase 3: intra-chunk product, output, state update
        bf16x8 vop[2][K::VB];
        if (MODE != WM_READOUT) {
#pragma unroll
            for (int ks = 0; ks < 2; ks++)
#pragma unroll
                for (int vb = 0; vb < K::VB; vb++)
                    vop[ks][vb] = load8(sVT + (16 * (w * K::VB + vb) + r16) * K::RC + 32 * ks + 8 * g);
        }
        if (MODE == WM_CAUSAL) {
#pragma unroll
            for (int ib = 0; ib < 4; ib++)
#pragma unroll
                for (int ks = 0; ks <= ib / 2; ks++) {
                    const bf16x8 a = load8(sA + (16 * ib + r16) * K::RC + 32 * ks + 8 * g);
#pragma unroll
                    for (int vb = 0; vb < K::VB; vb++) num[ib][vb] = mfma_bf16(a, vop[ks][vb], num[ib][vb]);
                }
        }
        if (MODE != WM_STATE) {
            bf16_t *yb = p.y + base + (size_t)t0 * D;
#pragma unroll
            for (int ib = 0; ib < 4; ib++) {
                const int i0 = 16 * ib + 4 * g;
                f32x4 den = zero4();
                const int nparts = (MODE == WM_CAUSAL) ? K::NW + 1 : K::NW;
                for (int pw = 0; pw < nparts; pw++) {
                    const f32x4 dp = *reinterpret_cast<const f32x4 *>(sDen + pw * K::C + i0);
                    den += dp;
                }
#pragma unroll
                for (int vb = 0; vb < K::VB; vb++) {
                    const int n = 16 * (w * K::VB + vb) + r16;
#pragma unroll
                    for (int r = 0; r < 4; r++)
                        if (i0 + r < valid) yb[(size_t)(i0 + r) * D + n] = float_to_bf16_bits(num[ib][vb][r] / den[r]);
                }
            }
        }
        if (MODE != WM_READOUT) {
#pragma unroll
            for (int fb = 0; fb < K::FB; fb++)
#pragma unroll
                for (int ks = 0; ks < 2; ks++) {
                    const bf16x8 a = load8(sPKT + (16 * fb + r16) * K::RC + 32 * ks + 8 * g);
#pragma unroll
                    for (int vb = 0; vb < K::VB; vb++) sacc[fb][vb] = mfma_bf16(a, vop[ks][vb], sacc[fb][vb]);
                }
#pragma unroll
            for (int zb = 0; zb < K::ZB; zb++)
#pragma unroll
                for (int ks = 0; ks < 2; ks++) {
                    const int fb = w * K::ZB + zb;
                    const bf16x8 a = load8(sPKT + (16 * fb + r16) * K::RC + 32 * ks + 8 * g);
                    zacc[zb] = mfma_bf16(a, ones, zacc[zb]);
                }
        }
        __syncthreads();
    }

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
        for (int fb = 0; fb < K::FB; fb++)
#pragma unroll
            for (int vb = 0; vb < K::VB; vb++) {
                const int n = 16 * (w * K::VB + vb) + r16;
#pragma unroll
                for (int r = 0; r < 4; r++) So[(size_t)(16 * fb + 4 * g + r) * D + n] = sacc[fb][vb][r];
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
__global__ __launch_bounds__(WideCfg<D>::NT, 1) void fm_hedgehog_kernel(const bf16_t *__restrict__ x,
                                                                        const bf16_t *__restrict__ W,
                                                                        const bf16_t *__restrict__ b,
                                                                        bf16_t *__restrict__ phi, int H, int N,
                                                                        int cpw, int wg_per_bh) {
    using K = WideCfg<D>;
    __shared__ __attribute__((aligned(16))) bf16_t sPhi[K::C * K::RQ];
    const int tid = threadIdx.x;
    const int w = tid >> 6, lane = tid & 63, g = lane >> 4, r16 = lane & 15;
    const int bh = blockIdx.x / wg_per_bh, part = blockIdx.x % wg_per_bh;
    const int h = bh % H;
    bf16x8 wA[K::LB][K::KSD];
    float bl2[K::LB][4];
    load_directions<D>(W, b, h, w, g, r16, wA, bl2);
    const bf16_t *xh = x + (size_t)bh * N * D;
    bf16_t *ph = phi + (size_t)bh * N * K::DP;
    for (int c = 0; c < cpw; c++) {
        const int t0 = (part * cpw + c) * K::C;
        if (t0 >= N) break;
        const int valid = min(K::C, N - t0);
        phi_chunk<D, false, true, false>(xh, t0, valid, wA, bl2, w, g, r16, sPhi, nullptr);
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
    return n < 1 ? 1 : (n > 4 ? 4 : n);
}

}  // namespace hh
