// hh_narrow.hip -- chunked causal / bidirectional attention with the degree-2 Taylor map,
// head dim 16, on the CDNA4 matrix cores (bf16 in, fp32 state).
//
// The Taylor map phi(x) = [1, x, x_a x_c / sqrt(2)] makes phi(q)^T phi(k) = 1 + s + s^2/2
// with s = q.k exactly (paper-graph-ui walkthrough of "The Hedgehog & the Porcupine",
// section 3.4, "The Taylor Exponential as a Bridge Result").  The same kernels run the
// generalised quadratic p(s) = a + b s + c s^2 of the learned global quadratic (paperlayer.ai
// summary of arXiv 2610.13674, section 2 and App. D): the map [sqrt a, sqrt b x, sqrt c x_a x_c]
// with per-head coefficients, of which the Taylor map is the case (1, 1, 1/2).  Every feature
// block takes its coefficient's root as a scale and the closed form below uses a, b, c.  The chunk recurrence is the
// same regrouping of Eq. 2 as in the Hedgehog kernels:
//     y_c = (phiQ_c Sp + A_c V_c) / (phiQ_c zp + A_c 1),  A_c = tril(phiQ_c phiK_c^T)
//     Sp += phiK_c^T V_c,  zp += phiK_c^T 1
// Two choices specific to this map:
//   * The intra-chunk kernel matrix A_c is formed from the closed form a + b s + c s^2
//     with s = Q_c K_c^T (a K = 16 product), the identity above, instead of a K = 273
//     product of feature vectors.
//   * Features are never stored: each lane builds the 8 feature values an MFMA operand
//     slot needs from the raw q or k values, so two waves hold the whole state in registers.
//   * The state is kept in a packed symmetric basis.  phi(q)^T phi(k) only involves the
//     quadratic features through sum_{a,c} q_a q_c k_a k_c / 2, in which the pairs (a, c) and
//     (c, a) contribute equally; so one feature per unordered pair carries both: x_a x_c for
//     a != c, x_a^2 / sqrt(2) on the diagonal.  1 + 16 + 136 = 153 features (padded to 160)
//     give the same phi(q)^T phi(k) as the 273 canonical ones, and the canonical state is
//     recovered exactly: S_ac = S_ca = (packed row {a,c}) / sqrt(2) off the diagonal.
// Internal feature-row order: block 0 = x_p; block 1 + o (o = 0..7) = the pair (p, p + o mod
// 16) for p = 0..15 (o = 0: the diagonal); block 9 = the pairs (p, p + 8) for p < 8, the
// constant 1 at p = 8, zero rows at p > 8.  Every unordered pair appears exactly once.
#include "hh_common.h"
#include "hh_kernels.h"

namespace hh {

namespace {
constexpr int D = 16;
constexpr int C = 64;
constexpr int FB = 10;          // 16-row feature blocks (160 rows)
constexpr int KSF = FB / 2;     // 32-wide K steps over features
constexpr int RR = D + 8;       // row stride of [C][D] tiles (bf16)
constexpr int RT = C + 8;       // row stride of [D][C] tiles (bf16)
constexpr int QFP = D + 8;      // row stride of the fp32 [C][D] query tile: 96 bytes, so the 16-byte
                                // reads of 16 rows x 4 column runs hit distinct banks
constexpr int KTP = C + 8;      // row stride of the fp32 [D][C] key tile: 288 bytes (32 mod 256)
// A zero state of one slot: the starting state read when the caller gives none, so that its
// loads are unconditional and leave together (a test of the pointer per element would wait on
// each load before issuing the next).
__device__ float zero_slot[kTaylorRowsInternal * (D + 1)];
constexpr float kInvSqrt2 = 0.70710678118654752f;
enum { NM_STATE = 0, NM_CAUSAL = 1, NM_READOUT = 2 };
}  // namespace

// Packed feature of internal block fb at position 4 g + r of a token, from the token's values
// rotated by the lane group: x[j] = value (4 g + j) mod 16.  m9 = (g < 2), c9 = (g == 2) select
// block 9's pair rows, its constant and its zero rows.  qc scales the constant, linear, diagonal
// and off-diagonal features (for the Taylor map 1, 1, 1/sqrt 2 and 1).
__device__ __forceinline__ float packed_feature(int fb, int r, const float (&x)[12], float m9, float c9,
                                                const QuadCoef &qc) {
    if (fb == 0) return x[r] * qc.sb;
    if (fb == 1) return x[r] * x[r] * qc.sc;
    if (fb < 9) return x[r] * x[r + fb - 1] * qc.s2c;
    return r == 0 ? fmaf(x[0] * x[8] * qc.s2c, m9, c9 * qc.sa) : x[r] * x[r + 8] * qc.s2c * m9;
}

// Work of wave H of the two waves of a workgroup.  Wave H holds the state rows of the K steps
// [KS0, KS1) (feature blocks 2 KS0 .. 2 KS1 - 1): wave 0 steps 0-2, wave 1 steps 3-4 plus the
// intra-chunk part, so each wave builds only its own feature operands.  The read-out partials
// over the two halves meet in LDS: each wave finishes two of the four 16-token blocks.  GQ: the
// generalised quadratic map (coefficients per head); otherwise the Taylor map, whose scales are
// compile-time constants.
template <int MODE, int H, bool GQ>
__device__ __forceinline__ void narrow_wave(const NarrowParams &p, int bh, int s, int lane, bf16_t *sQ, bf16_t *sK,
                                            float *sQf, float *sKTf, bf16_t *sVT, f32x4 *sX) {
    constexpr int KS0 = H == 0 ? 0 : 3, KS1 = H == 0 ? 3 : KSF;
    constexpr int NB = 2 * (KS1 - KS0);  // feature blocks held by this wave
    constexpr int FB0 = 2 * KS0;
    const int g = lane >> 4, r16 = lane & 15;
    const int t_begin = s * p.seg_len;
    const int t_end = min(p.N, t_begin + p.seg_len);
    const size_t base = (size_t)bh * p.N * D;

    // State S[f][n] (lane: column n = r16, rows f = 16 fb + 4 g + r) and z (same rows, every column).
    f32x4 sacc[NB], zacc[NB];
    {
        const float *Si = zero_slot, *zi = zero_slot + kTaylorRowsInternal * D;
        if (MODE != NM_STATE && p.S_in) {
            const size_t slot = (size_t)bh * p.in_bh_stride + (size_t)s * p.in_seg_stride;
            Si = p.S_in + slot * kTaylorRowsInternal * D;
            zi = p.z_in + slot * kTaylorRowsInternal;
        }
#pragma unroll
        for (int lb = 0; lb < NB; lb++)
#pragma unroll
            for (int r = 0; r < 4; r++) {
                const int f = 16 * (FB0 + lb) + 4 * g + r;
                sacc[lb][r] = Si[(size_t)f * D + r16];
                zacc[lb][r] = zi[f];
            }
    }
    const bf16x8 ones = ones_bf16x8();
    const float m9 = g < 2 ? 1.0f : 0.0f, c9 = g == 2 ? 1.0f : 0.0f;          // query side, block 9
    const float m9k = r16 < 8 ? 1.0f : 0.0f;                                    // key side, block 9
    const QuadCoef qc = GQ ? quad_coef(p.coef, bh % p.H) : quad_coef(nullptr, 0);

    // Chunk inputs (lane = token) are fetched into registers one chunk ahead, so their memory
    // latency overlaps the previous chunk's work: wave 0 q, k, v, wave 1 k.
    bf16x8 pq[2], pk[2], pv[2];
    auto fetch = [&](int tc) {
        const bool ok = tc + lane < t_end;
        const bf16_t *qr = p.q + base + (size_t)(tc + lane) * D;
        const bf16_t *kr = p.k + base + (size_t)(tc + lane) * D;
        const bf16_t *vr = p.v + base + (size_t)(tc + lane) * D;
#pragma unroll
        for (int hlf = 0; hlf < 2; hlf++) {
            if (H == 0) {
                pq[hlf] = (ok && MODE != NM_STATE) ? load8(qr + 8 * hlf) : zero_bf16x8();
                pk[hlf] = (ok && MODE == NM_CAUSAL) ? load8(kr + 8 * hlf) : zero_bf16x8();
                pv[hlf] = (ok && MODE != NM_READOUT) ? load8(vr + 8 * hlf) : zero_bf16x8();
            } else {
                pk[hlf] = (ok && MODE != NM_READOUT) ? load8(kr + 8 * hlf) : zero_bf16x8();
            }
        }
    };
    // The segment-state pass takes the chunks last to first (its sum does not depend on the
    // order), so that the segment's first chunks are the ones still in L2 when the causal pass,
    // which starts with them, begins.  Step k handles the chunk at chunk_t0(k).
    const int nch = t_end > t_begin ? (t_end - t_begin + C - 1) / C : 0;
    auto chunk_t0 = [&](int k) { return t_begin + C * (MODE == NM_STATE ? nch - 1 - k : k); };
    if (nch > 0) fetch(chunk_t0(0));

    for (int k = 0; k < nch; k++) {
        const int t0 = chunk_t0(k);
        const int valid = min(C, t_end - t0);
        // ---- stage the chunk: wave 0 q in fp32 (feature values) and, for the intra-chunk
        // products, q and k in bf16, and v transposed; wave 1 k transposed in fp32 (tokens
        // contiguous).  Feature values are formed in fp32, so the tiles they come from hold fp32.
        {
            const int j = lane;
            if (H == 0) {
                if (MODE == NM_CAUSAL) {
#pragma unroll
                    for (int hlf = 0; hlf < 2; hlf++) {
                        store8(sQ + j * RR + 8 * hlf, pq[hlf]);
                        store8(sK + j * RR + 8 * hlf, pk[hlf]);
                    }
                }
                if (MODE != NM_STATE) {
#pragma unroll
                    for (int m4 = 0; m4 < D / 4; m4++) {
                        f32x4 f;
#pragma unroll
                        for (int r = 0; r < 4; r++) f[r] = (float)pq[m4 / 2][4 * (m4 % 2) + r];
                        *reinterpret_cast<f32x4 *>(sQf + j * QFP + 4 * m4) = f;
                    }
                }
                if (MODE != NM_READOUT) {
#pragma unroll
                    for (int m = 0; m < D; m++) reinterpret_cast<__bf16 *>(sVT)[m * RT + j] = pv[m / 8][m % 8];
                }
            } else if (MODE != NM_READOUT) {
#pragma unroll
                for (int m = 0; m < D; m++) sKTf[m * KTP + j] = (float)pk[m / 8][m % 8];
            }
        }
        __syncthreads();
        if (k + 1 < nch) fetch(chunk_t0(k + 1));

        // V as a B operand, K = tokens in the order of two stacked accumulator blocks:
        // slot s < 4 -> j = 32 ks + 4 g + s, slot s >= 4 -> j = 32 ks + 16 + 4 g + s - 4.
        bf16x8 vop[2];
        if (MODE != NM_READOUT) {
#pragma unroll
            for (int ks = 0; ks < 2; ks++) {
                const bf16_t *vp = sVT + r16 * RT + 32 * ks + 4 * g;
                vop[ks] = cat(load4(vp), load4(vp + 16));
            }
        }

        if (MODE != NM_STATE) {
            f32x4 num[4], den[4];
#pragma unroll
            for (int ib = 0; ib < 4; ib++) {
                num[ib] = zero4();
                den[ib] = zero4();
            }
            // ---- read-out against the carried state over this wave's K steps; phi(q) built per
            // operand slot
#pragma unroll
            for (int ib = 0; ib < 4; ib++) {
                const int i = 16 * ib + r16;
                // the token's values rotated by the lane group, as far as this wave's blocks reach
                constexpr int NRUN = H == 0 ? 2 : 3;
                float x[12];
#pragma unroll
                for (int m = 0; m < 12; m++) x[m] = 0.0f;
#pragma unroll
                for (int m = 0; m < NRUN; m++) {
                    const f32x4 q4 = *reinterpret_cast<const f32x4 *>(sQf + i * QFP + 4 * ((g + m) & 3));
#pragma unroll
                    for (int r = 0; r < 4; r++) x[4 * m + r] = q4[r];
                }
#pragma unroll
                for (int ks = KS0; ks < KS1; ks++) {
                    bf16x8 a;
#pragma unroll
                    for (int r = 0; r < 4; r++) {
                        a[r] = (__bf16)packed_feature(2 * ks, r, x, m9, c9, qc);
                        a[4 + r] = (__bf16)packed_feature(2 * ks + 1, r, x, m9, c9, qc);
                    }
                    const int lb = 2 * (ks - KS0);
                    num[ib] = mfma_bf16(a, acc_pair_to_operand(sacc[lb], sacc[lb + 1]), num[ib]);
                    den[ib] = mfma_bf16(a, acc_pair_to_operand(zacc[lb], zacc[lb + 1]), den[ib]);
                }
            }
            // ---- intra-chunk part (causal, wave 1): A = a + b s + c s^2 on j <= i, s = k_j . q_i
            if (MODE == NM_CAUSAL && H == 1) {
                // keys past the end of the chunk count in no row sum (their v rows are zero)
                bf16x8 onesv[2];
#pragma unroll
                for (int ks = 0; ks < 2; ks++)
#pragma unroll
                    for (int sl = 0; sl < 8; sl++) {
                        const int j = 32 * ks + (sl < 4 ? 4 * g + sl : 16 + 4 * g + sl - 4);
                        onesv[ks][sl] = (__bf16)(j < valid ? 1.0f : 0.0f);
                    }
                // causal mask of the diagonal blocks: key 4 g + r of the block against query r16
                float cm[4];
#pragma unroll
                for (int r = 0; r < 4; r++) cm[r] = 4 * g + r <= r16 ? 1.0f : 0.0f;
                bf16x8 kop[4], qop[4];
#pragma unroll
                for (int b = 0; b < 4; b++) {
                    kop[b] = g < 2 ? load8(sK + (16 * b + r16) * RR + 8 * g) : zero_bf16x8();
                    qop[b] = g < 2 ? load8(sQ + (16 * b + r16) * RR + 8 * g) : zero_bf16x8();
                }
#pragma unroll
                for (int ib = 0; ib < 4; ib++) {
                    f32x4 at[4];
#pragma unroll
                    for (int jb = 0; jb < 4; jb++) {
                        if (jb <= ib) {
                            const f32x4 sdot = mfma_bf16(kop[jb], qop[ib], zero4());
                            // sdot: lane holds i = 16 ib + r16, j = 16 jb + 4 g + r
#pragma unroll
                            for (int r = 0; r < 4; r++) {
                                const float sv = sdot[r];
                                const float av = fmaf(sv, fmaf(qc.c, sv, qc.b), qc.a);
                                at[jb][r] = jb < ib ? av : av * cm[r];
                            }
                        } else {
                            at[jb] = zero4();
                        }
                    }
#pragma unroll
                    for (int ks = 0; ks <= ib / 2; ks++) {
                        const bf16x8 a = acc_pair_to_operand(at[2 * ks], at[2 * ks + 1]);
                        num[ib] = mfma_bf16(a, vop[ks], num[ib]);
                        den[ib] = mfma_bf16(a, onesv[ks], den[ib]);
                    }
                }
            }
            // ---- partials for the other wave's token blocks go through LDS; this wave finishes
            // token blocks 2 H, 2 H + 1
#pragma unroll
            for (int ibl = 0; ibl < 2; ibl++) {
                const int ib = 2 * (1 - H) + ibl;
                sX[((H * 2 + ibl) * 2 + 0) * 64 + lane] = num[ib];
                sX[((H * 2 + ibl) * 2 + 1) * 64 + lane] = den[ib];
            }
            __syncthreads();
            bf16_t *yb = p.y + base + (size_t)t0 * D;
#pragma unroll
            for (int ibl = 0; ibl < 2; ibl++) {
                const int ib = 2 * H + ibl;
                const f32x4 on = sX[(((1 - H) * 2 + ibl) * 2 + 0) * 64 + lane];
                const f32x4 od = sX[(((1 - H) * 2 + ibl) * 2 + 1) * 64 + lane];
#pragma unroll
                for (int r = 0; r < 4; r++) {
                    const int i = 16 * ib + 4 * g + r;
                    if (i < valid)
                        yb[(size_t)i * D + r16] =
                            float_to_bf16_bits((num[ib][r] + on[r]) * __builtin_amdgcn_rcpf(den[ib][r] + od[r]));
                }
            }
        }

        if (MODE != NM_READOUT) {
            // ---- state update: phi(k)^T built per operand slot (rows: position p = r16 of each
            // block, K = tokens); the pair partner of p in block 1 + o is row (p + o) mod 16 of
            // the transposed key tile
            float kr[2][8], krs[2][8], okc[2][8];
#pragma unroll
            for (int ks = 0; ks < 2; ks++) {
                const float *kp = sKTf + r16 * KTP + 32 * ks + 4 * g;
                const f32x4 lo = *reinterpret_cast<const f32x4 *>(kp), hi = *reinterpret_cast<const f32x4 *>(kp + 16);
#pragma unroll
                for (int r = 0; r < 4; r++) {
                    kr[ks][r] = lo[r];
                    kr[ks][4 + r] = hi[r];
                    krs[ks][r] = kr[ks][r] * qc.sc;
                    krs[ks][4 + r] = kr[ks][4 + r] * qc.sc;
                    const int jlo = 32 * ks + 4 * g + r, jhi = jlo + 16;
                    okc[ks][r] = (r16 == 8 && jlo < valid) ? qc.sa : 0.0f;
                    okc[ks][4 + r] = (r16 == 8 && jhi < valid) ? qc.sa : 0.0f;
                }
            }
#pragma unroll
            for (int lb = 0; lb < NB; lb++)
#pragma unroll
                for (int ks = 0; ks < 2; ks++) {
                    const int fb = FB0 + lb;
                    bf16x8 a;
                    if (fb == 0) {
#pragma unroll
                        for (int sl = 0; sl < 8; sl++) a[sl] = (__bf16)(kr[ks][sl] * qc.sb);
                    } else if (fb == 1) {
#pragma unroll
                        for (int sl = 0; sl < 8; sl++) a[sl] = (__bf16)(kr[ks][sl] * krs[ks][sl]);
                    } else {
                        const int o = fb < 9 ? fb - 1 : 8;
                        const float *kp = sKTf + ((r16 + o) & 15) * KTP + 32 * ks + 4 * g;
                        const f32x4 lo = *reinterpret_cast<const f32x4 *>(kp);
                        const f32x4 hi = *reinterpret_cast<const f32x4 *>(kp + 16);
#pragma unroll
                        for (int r = 0; r < 4; r++) {
                            const float plo = lo[r] * kr[ks][r] * qc.s2c, phi_ = hi[r] * kr[ks][4 + r] * qc.s2c;
                            a[r] = (__bf16)(fb < 9 ? plo : fmaf(plo, m9k, okc[ks][r]));
                            a[4 + r] = (__bf16)(fb < 9 ? phi_ : fmaf(phi_, m9k, okc[ks][4 + r]));
                        }
                    }
                    sacc[lb] = mfma_bf16(a, vop[ks], sacc[lb]);
                    zacc[lb] = mfma_bf16(a, ones, zacc[lb]);
                }
        }
        __syncthreads();
    }

    // ---- segment end: this wave's rows
    float *So = nullptr, *zo = nullptr;
    bool canonical = false;
    if (MODE == NM_STATE) {
        const size_t slot = (size_t)bh * p.ws_bh_stride + s;
        So = p.S_ws + slot * kTaylorRowsInternal * D;
        zo = p.z_ws + slot * kTaylorRowsInternal;
    } else if (MODE == NM_CAUSAL && p.S_out && s == p.nseg_grid - 1) {
        So = p.S_out + (size_t)bh * 273 * D;
        zo = p.z_out + (size_t)bh * 273;
        canonical = true;
    }
    if (So && !canonical) {
#pragma unroll
        for (int lb = 0; lb < NB; lb++)
#pragma unroll
            for (int r = 0; r < 4; r++) {
                const int f = 16 * (FB0 + lb) + 4 * g + r;
                So[(size_t)f * D + r16] = sacc[lb][r];
                if (r16 == 0) zo[f] = zacc[lb][r];
            }
    } else if (So) {
        // canonical rows: 0 constant, 1 + a linear, 17 + 16 a + c the pair (a, c).  A packed pair
        // row splits into its two canonical rows, each 1/sqrt(2) of it; the antisymmetric part of
        // the caller's initial state, which the packed basis cannot hold (and which no output
        // depends on), is added back so that S_out = S0 + the sum over the keys exactly.
        const float *S0c = p.S0c ? p.S0c + (size_t)bh * 273 * D : nullptr;
        const float *z0c = p.z0c ? p.z0c + (size_t)bh * 273 : nullptr;
        // canonical rows of every element of this lane (-1: none); then the pair halves of the
        // initial state, all loaded before the first is used (from the output rows, masked, where
        // there is no initial state: a branch per element would wait on each load in turn)
        int cas[NB][4], cbs[NB][4];
#pragma unroll
        for (int lb = 0; lb < NB; lb++)
#pragma unroll
            for (int r = 0; r < 4; r++) {
                const int fb = FB0 + lb, pos = 4 * g + r;
                int ca = -1, cb = -1;
                if (fb == 0) {
                    ca = 1 + pos;
                } else if (fb == 1) {
                    ca = 17 + 17 * pos;
                } else if (fb < 9 || pos < 8) {
                    const int c = (pos + (fb < 9 ? fb - 1 : 8)) & 15;
                    ca = 17 + 16 * pos + c;
                    cb = 17 + 16 * c + pos;
                } else if (pos == 8) {
                    ca = 0;
                }
                cas[lb][r] = ca;
                cbs[lb][r] = cb;
            }
        const float *Ssrc = S0c ? S0c : So;
        const float *zsrc = z0c ? z0c : zo;
        float hs[NB][4], hz[NB][4];
#pragma unroll
        for (int lb = 0; lb < NB; lb++)
#pragma unroll
            for (int r = 0; r < 4; r++) {
                const int ca = cas[lb][r] < 0 ? 0 : cas[lb][r], cb = cbs[lb][r] < 0 ? 0 : cbs[lb][r];
                hs[lb][r] = Ssrc[(size_t)ca * D + r16] - Ssrc[(size_t)cb * D + r16];
                hz[lb][r] = zsrc[ca] - zsrc[cb];
            }
#pragma unroll
        for (int lb = 0; lb < NB; lb++)
#pragma unroll
            for (int r = 0; r < 4; r++) {
                const float sv = sacc[lb][r], zv = zacc[lb][r];
                const int ca = cas[lb][r], cb = cbs[lb][r];
                if (ca < 0) continue;
                if (cb < 0) {
                    So[(size_t)ca * D + r16] = sv;
                    if (r16 == 0) zo[ca] = zv;
                    continue;
                }
                // (selected, not scaled by zero: the stand-in rows may hold anything)
                const float h = S0c ? 0.5f * hs[lb][r] : 0.0f, hzz = z0c ? 0.5f * hz[lb][r] : 0.0f;
                const float sa = sv * kInvSqrt2 + h, sb = sv * kInvSqrt2 - h;
                const float za = zv * kInvSqrt2 + hzz, zb = zv * kInvSqrt2 - hzz;
                So[(size_t)ca * D + r16] = sa;
                So[(size_t)cb * D + r16] = sb;
                if (r16 == 0) {
                    zo[ca] = za;
                    zo[cb] = zb;
                }
            }
    }
}

template <int MODE, bool GQ>
__global__ __launch_bounds__(128, 2) void narrow_kernel(NarrowParams p) {
    __shared__ __attribute__((aligned(16))) bf16_t sQ[C * RR];
    __shared__ __attribute__((aligned(16))) bf16_t sK[C * RR];
    __shared__ __attribute__((aligned(16))) float sQf[C * QFP];
    __shared__ __attribute__((aligned(16))) float sKTf[D * KTP];
    __shared__ __attribute__((aligned(16))) bf16_t sVT[D * RT];
    __shared__ __attribute__((aligned(16))) f32x4 sX[2 * 2 * 2 * 64];  // read-out partials [wave][block][num, den][lane]
    const int bh = blockIdx.x / p.nseg_grid;
    const int s = blockIdx.x % p.nseg_grid;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    if (w == 0)
        narrow_wave<MODE, 0, GQ>(p, bh, s, lane, sQ, sK, sQf, sKTf, sVT, sX);
    else
        narrow_wave<MODE, 1, GQ>(p, bh, s, lane, sQ, sK, sQf, sKTf, sVT, sX);
}

hipError_t launch_narrow(int mode, const NarrowParams &p, int grid, hipStream_t st) {
    const bool gq = p.coef != nullptr;
    switch (mode) {
    case NM_STATE:
        if (gq) hipLaunchKernelGGL((narrow_kernel<NM_STATE, true>), dim3(grid), dim3(128), 0, st, p);
        else hipLaunchKernelGGL((narrow_kernel<NM_STATE, false>), dim3(grid), dim3(128), 0, st, p);
        break;
    case NM_CAUSAL:
        if (gq) hipLaunchKernelGGL((narrow_kernel<NM_CAUSAL, true>), dim3(grid), dim3(128), 0, st, p);
        else hipLaunchKernelGGL((narrow_kernel<NM_CAUSAL, false>), dim3(grid), dim3(128), 0, st, p);
        break;
    default:
        if (gq) hipLaunchKernelGGL((narrow_kernel<NM_READOUT, true>), dim3(grid), dim3(128), 0, st, p);
        else hipLaunchKernelGGL((narrow_kernel<NM_READOUT, false>), dim3(grid), dim3(128), 0, st, p);
        break;
    }
    return hipGetLastError();
}

}  // namespace hh
