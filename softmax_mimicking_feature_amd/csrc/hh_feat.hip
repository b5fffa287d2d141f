// hh_feat.hip -- feature-map variants and the linear-attention passes over given features.
//
// Feature maps of the walkthrough's section 3.4, "The Hedgehog MLP Feature Map", beyond the
// two-sided exponential map (which has its own fused kernels):
//   HH_MAP_EXP              phi_l = exp(w_l.x + b_l), d' = d        (Choice 1, default d' = d)
//   HH_MAP_SOFTMAX          phi_l = exp(w_l.x) / sum_i exp(w_i.x)   (Choice 4, no bias, d' = d)
//   HH_MAP_HEDGEHOG_SOFTMAX [softmax(W x), softmax(-W x)], d' = 2d   (Choice 4 with the negation
//                           mapping of Choice 3, one softmax per half)
// The softmax maps need every direction of a token before any feature is final, so they are
// computed by a feature-map kernel into a workspace, and the attention passes below read the
// features (bf16, the precision the matrix cores take them in) instead of q and k.
//
// Attention over given features (Eq. 2, section 2; running sums of section 3.4, "Complexity
// Analysis"), per 64-token chunk c with the state Sp, zp before it:
//     y_c = (phiQ_c Sp + tril(phiQ_c phiK_c^T) V_c) / (phiQ_c zp + tril(phiQ_c phiK_c^T) 1)
//     Sp += phiK_c^T V_c,  zp += phiK_c^T 1
// Modes: STATE (segment aggregates into fp32 slots), CAUSAL (from the segment's starting state),
// READOUT (bidirectional: against the total).  One wave per 16 value columns (d / 16 waves),
// each holding its columns of S for every feature in fp32 accumulators; the z rows are split
// over the waves.
#include "hh_common.h"
#include "hh_kernels.h"

namespace hh {

namespace {

enum { FM_STATE = 0, FM_CAUSAL = 1, FM_READOUT = 2 };

// Transposing LDS read (ds_read_b64_tr_b16): within each group of 16 lanes, lane i receives, in
// slot s, element i % 4 of the 4-element run that lane 4 s + i / 4 addresses.
typedef short i16x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ bf16x4 tr_read(const bf16_t *p) {
    const i16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4_t *)(p));
    return __builtin_bit_cast(bf16x4, v);
}

// MFMA operand whose K index runs down the rows of a row-major LDS tile: lane (g, r16) gets
// column c0 + r16, rows r0 + 8 g .. r0 + 8 g + 7.  `lane_off` = (8 g + r16 / 4) pitch + 4 (r16 % 4).
__device__ __forceinline__ bf16x8 down_rows(const bf16_t *tile, int lane_off, int r0, int c0, int pitch) {
    const bf16_t *p = tile + lane_off + r0 * pitch + c0;
    return cat(tr_read(p), tr_read(p + 4 * pitch));
}

// Tile row pitch in elements: rows start 32 bytes apart modulo 128 bytes (bank spread for the
// 8- and 16-byte row reads and the transposing reads), and 8-byte aligned.
constexpr int pitch_of(int n) { return n + (((16 - n) % 64) + 64) % 64; }

template <int D, int DP, int MODE>
struct FeatCfg {
    static constexpr int C = 64;                         // tokens per chunk
    static constexpr int NW = D / 16;                    // waves: one per 16 value columns
    static constexpr int NT = 64 * NW;
    static constexpr int DPP = (DP + 31) / 32 * 32;      // features padded to whole K steps
    static constexpr int FB = DPP / 16;                  // 16-row feature blocks of S
    static constexpr int KSF = DPP / 32;                 // K steps over the features
    static constexpr int ZB = FB / NW;                   // z blocks per wave (1 or 2)
    static constexpr int PF = pitch_of(DPP), PV = pitch_of(D), PA = pitch_of(C);
    static constexpr bool USE_Q = MODE != FM_STATE;
    static constexpr bool USE_K = MODE != FM_READOUT;
    static constexpr int SZ_F = C * PF * 2, SZ_V = C * PV * 2, SZ_A = C * PA * 2;
    static constexpr int OFF_Q = 0;
    static constexpr int OFF_K = OFF_Q + (USE_Q ? SZ_F : 0);
    static constexpr int OFF_V = OFF_K + (USE_K ? SZ_F : 0);
    static constexpr int OFF_A = OFF_V + (USE_K ? SZ_V : 0);
    static constexpr int OFF_DEN = OFF_A + (MODE == FM_CAUSAL ? SZ_A : 0);  // [NW][C] partials, [4][C] row sums
    static constexpr int LDS_BYTES = OFF_DEN + (USE_Q ? (NW + 4) * C * 4 : 0);
    // 16-byte pieces of the next chunk each thread prefetches into registers
    static constexpr int PQ = USE_Q ? C * DP / 8 / NT : 0;
    static constexpr int PK = USE_K ? C * DP / 8 / NT : 0;
    static constexpr int PVV = USE_K ? C * D / 8 / NT : 0;
    static_assert(ZB == 1 || ZB == 2, "z rows split evenly over the waves");
    static_assert((!USE_Q || PQ * NT * 8 == C * DP) && (!USE_K || PVV * NT * 8 == C * D), "whole pieces per thread");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
};

// Registers holding the next chunk on its way into LDS.
template <int D, int DP, int MODE>
struct FeatPrefetch {
    using K = FeatCfg<D, DP, MODE>;
    bf16x8 q[K::PQ > 0 ? K::PQ : 1], k[K::PK > 0 ? K::PK : 1], v[K::PVV > 0 ? K::PVV : 1];
};

// piece p of a [C][n] row-major chunk: row p / (n / 8), columns 8 (p % (n / 8)) .. + 7; rows at or
// past `valid` are zero (keys past the end add nothing; their values and queries are unused).
template <int n>
__device__ __forceinline__ bf16x8 load_piece(const bf16_t *src, int p, int valid) {
    const int row = p / (n / 8), col = 8 * (p % (n / 8));
    return row < valid ? *reinterpret_cast<const bf16x8 *>(src + (size_t)row * n + col) : zero_bf16x8();
}
template <int n, int pitch>
__device__ __forceinline__ void store_piece(bf16_t *tile, int p, const bf16x8 &x) {
    const int row = p / (n / 8), col = 8 * (p % (n / 8));
    *reinterpret_cast<bf16x8 *>(tile + row * pitch + col) = x;
}

template <int D, int DP, int MODE>
__device__ __forceinline__ void feat_fetch(FeatPrefetch<D, DP, MODE> &pf, const FeatParams &p, size_t tok0, int valid,
                                           int tid) {
    using K = FeatCfg<D, DP, MODE>;
#pragma unroll
    for (int i = 0; i < K::PQ; i++) pf.q[i] = load_piece<DP>(p.phiq + tok0 * DP, tid + K::NT * i, valid);
#pragma unroll
    for (int i = 0; i < K::PK; i++) pf.k[i] = load_piece<DP>(p.phik + tok0 * DP, tid + K::NT * i, valid);
#pragma unroll
    for (int i = 0; i < K::PVV; i++) pf.v[i] = load_piece<D>(p.v + tok0 * D, tid + K::NT * i, valid);
}

// phi(q) is kept in LDS in the reordered column order of qperm_pos (hh_common.h), so that the
// read-out and normaliser operands, in the K order of an accumulator pair, are 16-byte reads.
template <int n, int pitch>
__device__ __forceinline__ void store_piece_qperm(bf16_t *tile, int p, const bf16x8 &x) {
    const int row = p / (n / 8), col = 8 * (p % (n / 8));
    store8_qperm(tile + row * pitch, col, x);
}

template <int D, int DP, int MODE>
__device__ __forceinline__ void feat_commit(const FeatPrefetch<D, DP, MODE> &pf, unsigned char *smem, int tid) {
    using K = FeatCfg<D, DP, MODE>;
#pragma unroll
    for (int i = 0; i < K::PQ; i++)
        store_piece_qperm<DP, K::PF>(reinterpret_cast<bf16_t *>(smem + K::OFF_Q), tid + K::NT * i, pf.q[i]);
#pragma unroll
    for (int i = 0; i < K::PK; i++)
        store_piece<DP, K::PF>(reinterpret_cast<bf16_t *>(smem + K::OFF_K), tid + K::NT * i, pf.k[i]);
#pragma unroll
    for (int i = 0; i < K::PVV; i++)
        store_piece<D, K::PV>(reinterpret_cast<bf16_t *>(smem + K::OFF_V), tid + K::NT * i, pf.v[i]);
}

// Workgroup -> (sequence bh, segment s); with BH a multiple of 8, all segments of a sequence
// land on one XCD (workgroups are dealt to the eight XCDs round-robin).
__device__ __forceinline__ void feat_head_segment(int nseg, int &bh, int &s) {
    const int b = blockIdx.x, BH = gridDim.x / nseg;
    if (BH % 8 == 0) {
        const int j = b >> 3;
        bh = (b & 7) + 8 * (j / nseg);
        s = j % nseg;
    } else {
        bh = b / nseg;
        s = b % nseg;
    }
}

// Slot image: lane L of wave w holds S blocks (fb, w) for every fb; blocks 2 j, 2 j + 1 are
// piece w FB / 2 + j, halves 0 and 1, at f32x4 index (2 e + h) 64 + L.
__device__ __forceinline__ f32x4 *fslot(float *S, int e, int h, int L) {
    return reinterpret_cast<f32x4 *>(S) + (2 * e + h) * 64 + L;
}

template <int D, int DP, int MODE>
__device__ void feat_body(const FeatParams &p, unsigned char *smem, int bh, int s) {
    using K = FeatCfg<D, DP, MODE>;
    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, g = lane >> 4, r16 = lane & 15;
    const int t_begin = s * p.seg_len;
    const int t_end = min(p.N, t_begin + p.seg_len);
    const int n = t_end > t_begin ? (t_end - t_begin + K::C - 1) / K::C : 0;
    const size_t tok_base = (size_t)bh * p.N;
    bf16_t *sQ = reinterpret_cast<bf16_t *>(smem + K::OFF_Q);
    bf16_t *sK = reinterpret_cast<bf16_t *>(smem + K::OFF_K);
    bf16_t *sV = reinterpret_cast<bf16_t *>(smem + K::OFF_V);
    bf16_t *sA = reinterpret_cast<bf16_t *>(smem + K::OFF_A);
    float *sDen = reinterpret_cast<float *>(smem + K::OFF_DEN);   // [NW][C] partials
    float *sRS = sDen + K::NW * K::C;                              // [4][C] intra-chunk row sums

    // Feature columns DP .. DPP - 1 of the tiles and the never-written upper score blocks stay
    // zero; so do the row sums of blocks above the diagonal.
    for (int i = tid; i < K::LDS_BYTES / 16; i += K::NT) reinterpret_cast<f32x4 *>(smem)[i] = zero4();
    __syncthreads();

    // ---- starting state: S block (fb, w) rows 16 fb + 4 g + r, value column 16 w + r16
    f32x4 sacc[K::FB];
    f32x4 zacc[K::ZB];  // z blocks ZB w + zb (every column holds the same value)
#pragma unroll
    for (int fb = 0; fb < K::FB; fb++) sacc[fb] = zero4();
#pragma unroll
    for (int zb = 0; zb < K::ZB; zb++) zacc[zb] = zero4();
    if (MODE == FM_CAUSAL && p.S0) {
        const float *S0 = p.S0 + (size_t)bh * DP * D;
        const float *z0 = p.z0 + (size_t)bh * DP;
#pragma unroll
        for (int fb = 0; fb < K::FB; fb++)
#pragma unroll
            for (int r = 0; r < 4; r++) {
                const int row = 16 * fb + 4 * g + r;
                if (row < DP) sacc[fb][r] = S0[(size_t)row * D + 16 * w + r16];
            }
#pragma unroll
        for (int zb = 0; zb < K::ZB; zb++)
#pragma unroll
            for (int r = 0; r < 4; r++) {
                const int row = 16 * (K::ZB * w + zb) + 4 * g + r;
                if (row < DP) zacc[zb][r] = z0[row];
            }
    }
    if (MODE != FM_STATE) {
        // slots to add: the exclusive prefix (mode 1), the total (mode 2), or the aggregates of
        // every earlier segment (mode 3, summed here)
        int t0 = 0, t1 = 0;
        if (p.slot_mode == 1 && s > 0) t0 = s, t1 = s + 1;
        if (p.slot_mode == 2) t0 = 0, t1 = 1;
        if (p.slot_mode == 3) t0 = 0, t1 = s;
        for (int t = t0; t < t1; t++) {
            const size_t sl = (size_t)bh * p.slot_bh_stride + t;
            float *img = p.S_slots + sl * K::DPP * D;
#pragma unroll
            for (int j = 0; j < K::FB / 2; j++) {
                sacc[2 * j] += *fslot(img, w * (K::FB / 2) + j, 0, lane);
                sacc[2 * j + 1] += *fslot(img, w * (K::FB / 2) + j, 1, lane);
            }
            const float *zs = p.z_slots + sl * K::DPP;
#pragma unroll
            for (int zb = 0; zb < K::ZB; zb++)
                zacc[zb] += *reinterpret_cast<const f32x4 *>(zs + 16 * (K::ZB * w + zb) + 4 * g);
        }
    }

    FeatPrefetch<D, DP, MODE> pf;
    if (n > 0) {
        feat_fetch<D, DP, MODE>(pf, p, tok_base + t_begin, min(K::C, t_end - t_begin), tid);
        feat_commit<D, DP, MODE>(pf, smem, tid);
    }
    __syncthreads();

    const bf16x8 ones = ones_bf16x8();
    const int lane_tr = (8 * g + (r16 >> 2));  // row part of the transposing-read lane offset
    const int lane_trc = 4 * (r16 & 3);        // column part
    bf16_t *ybase = p.y + tok_base * D;

    for (int c = 0; c < n; c++) {
        const int t0 = t_begin + K::C * c;
        const int valid = min(K::C, t_end - t0);
        if (c + 1 < n) feat_fetch<D, DP, MODE>(pf, p, tok_base + t0 + K::C, min(K::C, t_end - t0 - K::C), tid);

        if (MODE != FM_STATE) {
            // ---- intra-chunk scores (causal): blocks (ib, jb <= ib) dealt over the waves; out[key][query]
            if (MODE == FM_CAUSAL) {
                for (int t = w; t < 10; t += K::NW) {
                    const int ib = t < 1 ? 0 : t < 3 ? 1 : t < 6 ? 2 : 3;
                    const int jb = t - ib * (ib + 1) / 2;
                    f32x4 a = zero4();
#pragma unroll
                    for (int ks = 0; ks < K::KSF; ks++) {
                        // K in the reordered feature order of the phi(q) tile
                        const bf16_t *krow = sK + (16 * jb + r16) * K::PF + 32 * ks;
                        const bf16x8 ko = cat(load4(krow + 4 * g), load4(krow + 16 + 4 * g));
                        const bf16x8 qo = *reinterpret_cast<const bf16x8 *>(sQ + (16 * ib + r16) * K::PF + 32 * ks + 8 * g);
                        a = mfma_bf16(ko, qo, a);
                    }
                    // lane: query 16 ib + r16, keys 16 jb + 4 g + r; keep key <= query
                    if (jb == ib) {
#pragma unroll
                        for (int r = 0; r < 4; r++)
                            if (4 * g + r > r16) a[r] = 0.0f;
                    }
                    const bf16x4 ab = to_bf16x4(a);
                    store4(sA + (16 * ib + r16) * K::PA + 16 * jb + 4 * g, ab);
                    float rs = ((float)ab[0] + (float)ab[1]) + ((float)ab[2] + (float)ab[3]);
                    rs += __shfl_xor(rs, 16);
                    rs += __shfl_xor(rs, 32);
                    if (g == 0) sRS[jb * K::C + 16 * ib + r16] = rs;
                }
            }
            // ---- partial denominators phiQ . zp over this wave's z blocks
#pragma unroll
            for (int ib = 0; ib < 4; ib++) {
                f32x4 dacc = zero4();
                if (K::ZB == 2) {
                    const bf16x8 zo = acc_pair_to_operand(zacc[0], zacc[K::ZB - 1]);
                    const bf16_t *row = sQ + (16 * ib + r16) * K::PF + 32 * w;
                    dacc = mfma_bf16(zo, *reinterpret_cast<const bf16x8 *>(row + 8 * g), dacc);
                } else {
                    // one block 16 w: the K step 32 (w / 2) with the other half zero
                    const f32x4 zz = zero4();
                    const bf16x8 zo = (w & 1) ? acc_pair_to_operand(zz, zacc[0]) : acc_pair_to_operand(zacc[0], zz);
                    const bf16_t *row = sQ + (16 * ib + r16) * K::PF + 32 * (w >> 1);
                    dacc = mfma_bf16(zo, *reinterpret_cast<const bf16x8 *>(row + 8 * g), dacc);
                }
                if (g == 0) sDen[w * K::C + 16 * ib + r16] = dacc[0];
            }
        }
        __syncthreads();

        // V operand of value block w for the two K steps over the chunk's keys (also the A
        // operand of the intra-chunk product: lane column = value column, K = keys)
        bf16x8 vop[2];
        if (MODE != FM_READOUT) {
#pragma unroll
            for (int ks = 0; ks < 2; ks++) vop[ks] = down_rows(sV, lane_tr * K::PV + lane_trc, 32 * ks, 16 * w, K::PV);
        }
        if (MODE != FM_STATE) {
            // ---- read-out (transposed: rows value columns, column query), intra product, output
            bf16x8 sop[K::KSF];
#pragma unroll
            for (int ks = 0; ks < K::KSF; ks++) sop[ks] = acc_pair_to_operand(sacc[2 * ks], sacc[2 * ks + 1]);
#pragma unroll
            for (int ib = 0; ib < 4; ib++) {
                const int i = 16 * ib + r16;
                f32x4 num = zero4();
                const bf16_t *row = sQ + i * K::PF;
#pragma unroll
                for (int ks = 0; ks < K::KSF; ks++)
                    num = mfma_bf16(sop[ks], *reinterpret_cast<const bf16x8 *>(row + 32 * ks + 8 * g), num);
                if (MODE == FM_CAUSAL) {
#pragma unroll
                    for (int ks = 0; ks <= ib / 2; ks++)
                        num = mfma_bf16(vop[ks], *reinterpret_cast<const bf16x8 *>(sA + i * K::PA + 32 * ks + 8 * g), num);
                }
                float den = 0.0f;
#pragma unroll
                for (int pw = 0; pw < K::NW; pw++) den += sDen[pw * K::C + i];
                if (MODE == FM_CAUSAL) {
#pragma unroll
                    for (int jb = 0; jb < 4; jb++) den += sRS[jb * K::C + i];
                }
                const float rd = __builtin_amdgcn_rcpf(den);
                f32x4 o;
#pragma unroll
                for (int r = 0; r < 4; r++) o[r] = num[r] * rd;
                if (i < valid) store4(ybase + (size_t)(t0 + i) * D + 16 * w + 4 * g, to_bf16x4(o));
            }
        }
        if (MODE != FM_READOUT) {
            // ---- state update with the chunk's keys: S += phiK^T V, z += phiK^T 1
#pragma unroll
            for (int ks = 0; ks < 2; ks++) {
#pragma unroll
                for (int fb = 0; fb < K::FB; fb++) {
                    const bf16x8 ko = down_rows(sK, lane_tr * K::PF + lane_trc, 32 * ks, 16 * fb, K::PF);
                    sacc[fb] = mfma_bf16(ko, vop[ks], sacc[fb]);
                }
#pragma unroll
                for (int zb = 0; zb < K::ZB; zb++) {
                    const bf16x8 ko = down_rows(sK, lane_tr * K::PF + lane_trc, 32 * ks, 16 * (K::ZB * w + zb), K::PF);
                    zacc[zb] = mfma_bf16(ko, ones, zacc[zb]);
                }
            }
        }
        __syncthreads();  // every wave is done with this chunk's tiles
        if (c + 1 < n) {
            feat_commit<D, DP, MODE>(pf, smem, tid);
            __syncthreads();
        }
    }

    if (MODE == FM_STATE) {
        const size_t sl = (size_t)bh * p.slot_bh_stride + s;
        float *img = p.S_slots + sl * K::DPP * D;
        if (p.slot_canonical) {  // [dpp][d] row-major, for the backward passes
#pragma unroll
            for (int fb = 0; fb < K::FB; fb++)
#pragma unroll
                for (int r = 0; r < 4; r++) img[(size_t)(16 * fb + 4 * g + r) * D + 16 * w + r16] = sacc[fb][r];
        } else {
#pragma unroll
            for (int j = 0; j < K::FB / 2; j++) {
                *fslot(img, w * (K::FB / 2) + j, 0, lane) = sacc[2 * j];
                *fslot(img, w * (K::FB / 2) + j, 1, lane) = sacc[2 * j + 1];
            }
        }
        float *zs = p.z_slots + sl * K::DPP;
        if (r16 == 0) {
#pragma unroll
            for (int zb = 0; zb < K::ZB; zb++)
                *reinterpret_cast<f32x4 *>(zs + 16 * (K::ZB * w + zb) + 4 * g) = zacc[zb];
        }
    } else if (MODE == FM_CAUSAL && p.S_out && s == p.nseg_grid - 1) {
        float *So = p.S_out + (size_t)bh * DP * D;
        float *zo = p.z_out + (size_t)bh * DP;
#pragma unroll
        for (int fb = 0; fb < K::FB; fb++)
#pragma unroll
            for (int r = 0; r < 4; r++) {
                const int row = 16 * fb + 4 * g + r;
                if (row < DP) So[(size_t)row * D + 16 * w + r16] = sacc[fb][r];
            }
        if (r16 == 0) {
#pragma unroll
            for (int zb = 0; zb < K::ZB; zb++)
#pragma unroll
                for (int r = 0; r < 4; r++) {
                    const int row = 16 * (K::ZB * w + zb) + 4 * g + r;
                    if (row < DP) zo[row] = zacc[zb][r];
                }
        }
    }
}

template <int D, int DP, int MODE>
__global__ __launch_bounds__(4 * D) void feat_kernel(FeatParams p) {  // one wave per 16 value columns
    __shared__ __attribute__((aligned(16))) unsigned char smem[FeatCfg<D, DP, MODE>::LDS_BYTES];
    int bh, s;
    feat_head_segment(p.nseg_grid, bh, s);
    feat_body<D, DP, MODE>(p, smem, bh, s);
}

// Segment scan over fp32 slots of `per` floats (S image, then z): mode 0 turns aggregates of
// slots 0 .. nseg-2 into exclusive prefixes in slots 1 .. nseg-1, mode 1 puts the total in slot 0.
__global__ void feat_scan_kernel(float *__restrict__ S, float *__restrict__ z, long perS, long perZ, int BH, int nseg,
                                 int mode) {
    const long idx = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (long)BH * (perS + perZ)) return;
    const long bh = idx / (perS + perZ), e = idx % (perS + perZ);
    float *base;
    long stride;
    if (e < perS) {
        base = S + bh * nseg * perS + e;
        stride = perS;
    } else {
        base = z + bh * nseg * perZ + (e - perS);
        stride = perZ;
    }
    // each thread loads eight slots before it adds or stores any, so its loads are in flight
    // together rather than one round trip per slot
    const int nin = mode == 0 ? nseg - 1 : nseg;
    float run = 0.0f;
    for (int t0 = 0; t0 < nin; t0 += 8) {
        float a[8];
#pragma unroll
        for (int i = 0; i < 8; i++) a[i] = t0 + i < nin ? base[(t0 + i) * stride] : 0.0f;
#pragma unroll
        for (int i = 0; i < 8; i++)
            if (t0 + i < nin) {
                if (mode == 0 && t0 + i > 0) base[(t0 + i) * stride] = run;
                run += a[i];
            }
    }
    base[mode == 0 ? (long)(nseg - 1) * stride : 0] = run;
}

// ---------------------------------------------------------------------------------------
// Feature maps with a W (maps 2, 3, 4) on the matrix cores, bf16.  One workgroup per
// kFmvBlocks x 64 tokens of one sequence; each wave loads the head's W operands into registers
// once and walks kFmvBlocks blocks of 16 tokens (the 16 tokens of an MFMA share its W rows, so
// they belong to one head).  u^T = W x^T for every direction (lane: token r16, directions
// 16 lb + 4 g + r), so that a token's d projections sit in its 4 lane groups and the softmax
// normaliser is two shuffles.  The next block's x is loaded while the current one is mapped.
constexpr int kFmvBlocks = 4;

template <int D, int MAP>
__global__ __launch_bounds__(256) void fm_variant_kernel(const bf16_t *__restrict__ x, const bf16_t *__restrict__ W,
                                                         const bf16_t *__restrict__ b, bf16_t *__restrict__ phi,
                                                         int tiles, int H, int N) {
    constexpr int LB = D / 16, KS = (D + 31) / 32;
    constexpr int DP = MAP == HH_MAP_HEDGEHOG_SOFTMAX_ ? 2 * D : D;
    const int lane = threadIdx.x & 63, g = lane >> 4, r16 = lane & 15;
    const long bh = blockIdx.x / tiles;
    const int n0 = (blockIdx.x % tiles) * 64 * kFmvBlocks + (threadIdx.x >> 6) * 16 + r16;
    const int h = (int)(bh % H);
    const bf16_t *Wh = W + (size_t)h * D * D;
    // the head's W through LDS once per workgroup (rows padded to 32 mod 256 bytes: the operand
    // reads of 16 rows x 4 column runs fall in distinct banks)
    constexpr int WP = D + 16;
    __shared__ __attribute__((aligned(16))) bf16_t sW[D * WP];
    stage_pieces<256, D * D / 8>(
        threadIdx.x, [&](int e) { return Wh + 8 * e; },
        [&](int e) { return sW + (e / (D / 8)) * WP + 8 * (e % (D / 8)); }, [](int) { return true; });
    __syncthreads();
    // A operands: W rows 16 lb + r16, input dims 32 ks + 8 g .. + 7 (D = 16: the upper half zero)
    bf16x8 wa[LB][KS];
#pragma unroll
    for (int lb = 0; lb < LB; lb++)
#pragma unroll
        for (int ks = 0; ks < KS; ks++)
            wa[lb][ks] = (32 * ks + 8 * g < D) ? *reinterpret_cast<const bf16x8 *>(sW + (16 * lb + r16) * WP + 32 * ks + 8 * g)
                                               : zero_bf16x8();
    float bl[LB][4];
#pragma unroll
    for (int lb = 0; lb < LB; lb++)
#pragma unroll
        for (int r = 0; r < 4; r++) bl[lb][r] = 0.0f;
    if (MAP == HH_MAP_EXP_ && b) {  // one test around the loads, so that they leave together
#pragma unroll
        for (int lb = 0; lb < LB; lb++)
#pragma unroll
            for (int r = 0; r < 4; r++) bl[lb][r] = bf16_bits_to_float(b[(size_t)h * D + 16 * lb + 4 * g + r]);
    }
    // B operand of a block: token r16, input dims 32 ks + 8 g .. + 7
    auto load_x = [&](int n, bf16x8 (&xb)[KS]) {
        const long tk = bh * N + (n < N ? n : 0);
#pragma unroll
        for (int ks = 0; ks < KS; ks++)
            xb[ks] = (32 * ks + 8 * g < D) ? *reinterpret_cast<const bf16x8 *>(x + (size_t)tk * D + 32 * ks + 8 * g)
                                           : zero_bf16x8();
    };
    bf16x8 xn[KS];
    load_x(n0, xn);
    for (int blk = 0; blk < kFmvBlocks; blk++) {
        const int n = n0 + 64 * blk;
        if (n - r16 >= N) break;  // the whole 16-token block lies past the end (wave-uniform)
        bf16x8 xb[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ks++) xb[ks] = xn[ks];
        if (blk + 1 < kFmvBlocks) load_x(n + 64, xn);
        const bool live = n < N;
        f32x4 u[LB];
#pragma unroll
        for (int lb = 0; lb < LB; lb++) {
            u[lb] = zero4();
#pragma unroll
            for (int ks = 0; ks < KS; ks++) u[lb] = mfma_bf16(wa[lb][ks], xb[ks], u[lb]);
        }
        // lane holds u of directions 16 lb + 4 g + r for token r16
        bf16_t *out = phi + (size_t)(bh * N + (live ? n : 0)) * DP;
        if (MAP == HH_MAP_EXP_) {
#pragma unroll
            for (int lb = 0; lb < LB; lb++) {
                f32x4 e;
#pragma unroll
                for (int r = 0; r < 4; r++) e[r] = exp2_fast((u[lb][r] + bl[lb][r]) * kLog2e);
                if (live) store4(out + 16 * lb + 4 * g, to_bf16x4(e));
            }
            continue;
        }
        // softmax over the d directions (and, two-sided, over their negations), in base 2: u is
        // scaled by log2(e) once for both halves
#pragma unroll
        for (int lb = 0; lb < LB; lb++)
#pragma unroll
            for (int r = 0; r < 4; r++) u[lb][r] *= kLog2e;
#pragma unroll
        for (int half = 0; half < (MAP == HH_MAP_HEDGEHOG_SOFTMAX_ ? 2 : 1); half++) {
            const float sg = half ? -1.0f : 1.0f;
            float mx = -INFINITY;
#pragma unroll
            for (int lb = 0; lb < LB; lb++)
#pragma unroll
                for (int r = 0; r < 4; r++) mx = fmaxf(mx, sg * u[lb][r]);
            mx = fmaxf(mx, __shfl_xor(mx, 16));
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            f32x4 e[LB];
            float sum = 0.0f;
#pragma unroll
            for (int lb = 0; lb < LB; lb++)
#pragma unroll
                for (int r = 0; r < 4; r++) {
                    e[lb][r] = exp2_fast(sg * u[lb][r] - mx);
                    sum += e[lb][r];
                }
            sum += __shfl_xor(sum, 16);
            sum += __shfl_xor(sum, 32);
            // the hardware reciprocal (about 1 ulp): the features are stored in bf16
            const float rs = __builtin_amdgcn_rcpf(sum);
#pragma unroll
            for (int lb = 0; lb < LB; lb++) {
                f32x4 o;
#pragma unroll
                for (int r = 0; r < 4; r++) o[r] = e[lb][r] * rs;
                if (live) store4(out + half * D + 16 * lb + 4 * g, to_bf16x4(o));
            }
        }
    }
}

// fp32 (and any dtype) feature map with a W on the vector units: one wave per token, lane l
// owns directions l and l + 64.
__global__ __launch_bounds__(256) void fm_variant_vec_kernel(int map, int dtype, int d, const void *x, const void *W,
                                                             const void *b, void *phi, long ntok, int H, int N) {
    const long tok = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (tok >= ntok) return;
    const int h = (int)((tok / N) % H);
    const int dp = map == HH_MAP_HEDGEHOG_SOFTMAX_ ? 2 * d : d;
    auto ldv = [&](const void *ptr, size_t i) {
        return dtype == HH_BF16_ ? bf16_bits_to_float(reinterpret_cast<const bf16_t *>(ptr)[i])
                                 : reinterpret_cast<const float *>(ptr)[i];
    };
    auto stv = [&](size_t i, float v) {
        if (dtype == HH_BF16_) reinterpret_cast<bf16_t *>(phi)[i] = float_to_bf16_bits(v);
        else reinterpret_cast<float *>(phi)[i] = v;
    };
    float u[2] = {0.0f, 0.0f};
#pragma unroll
    for (int j = 0; j < 2; j++) {
        const int l = lane + 64 * j;
        if (l < d) {
            float a = (map == HH_MAP_EXP_ && b) ? ldv(b, (size_t)h * d + l) : 0.0f;
            for (int m = 0; m < d; m++) a = fmaf(ldv(W, ((size_t)h * d + l) * d + m), ldv(x, (size_t)tok * d + m), a);
            u[j] = a;
        }
    }
    if (map == HH_MAP_EXP_) {
#pragma unroll
        for (int j = 0; j < 2; j++)
            if (lane + 64 * j < d) stv((size_t)tok * dp + lane + 64 * j, expf(u[j]));
        return;
    }
    for (int half = 0; half < (map == HH_MAP_HEDGEHOG_SOFTMAX_ ? 2 : 1); half++) {
        const float sg = half ? -1.0f : 1.0f;
        float mx = -INFINITY;
#pragma unroll
        for (int j = 0; j < 2; j++)
            if (lane + 64 * j < d) mx = fmaxf(mx, sg * u[j]);
        for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
        float e[2] = {0.0f, 0.0f}, sum = 0.0f;
#pragma unroll
        for (int j = 0; j < 2; j++)
            if (lane + 64 * j < d) {
                e[j] = expf(sg * u[j] - mx);
                sum += e[j];
            }
        for (int o = 32; o > 0; o >>= 1) sum += __shfl_xor(sum, o);
#pragma unroll
        for (int j = 0; j < 2; j++)
            if (lane + 64 * j < d) stv((size_t)tok * dp + half * d + lane + 64 * j, e[j] / sum);
    }
}

template <int D, int DP>
hipError_t launch_feat_d(int mode, const FeatParams &p, int grid, hipStream_t st) {
    switch (mode) {
    case FM_STATE: hipLaunchKernelGGL((feat_kernel<D, DP, FM_STATE>), dim3(grid), dim3(D * 4), 0, st, p); break;
    case FM_CAUSAL: hipLaunchKernelGGL((feat_kernel<D, DP, FM_CAUSAL>), dim3(grid), dim3(D * 4), 0, st, p); break;
    default: hipLaunchKernelGGL((feat_kernel<D, DP, FM_READOUT>), dim3(grid), dim3(D * 4), 0, st, p); break;
    }
    return hipGetLastError();
}

template <int D, int MAP>
hipError_t launch_fm_variant_d(const bf16_t *x, const bf16_t *W, const bf16_t *b, bf16_t *phi, long BH, int H, int N,
                               hipStream_t st) {
    const int tiles = (N + 64 * kFmvBlocks - 1) / (64 * kFmvBlocks);
    hipLaunchKernelGGL((fm_variant_kernel<D, MAP>), dim3((unsigned)(BH * tiles)), dim3(256), 0, st, x, W, b, phi, tiles,
                       H, N);
    return hipGetLastError();
}

}  // namespace

int feat_padded_dim(int dp) { return (dp + 31) / 32 * 32; }

int feat_wgs_per_cu(int d, int dp) {
    int lds = 0;
    switch (d * 1000 + dp) {
#define HH_FEAT_LDS(D, DP) \
    case D * 1000 + DP: lds = FeatCfg<D, DP, FM_CAUSAL>::LDS_BYTES; break;
        HH_FEAT_LDS(16, 16) HH_FEAT_LDS(16, 32) HH_FEAT_LDS(32, 32) HH_FEAT_LDS(32, 64)
        HH_FEAT_LDS(64, 64) HH_FEAT_LDS(64, 128) HH_FEAT_LDS(128, 128) HH_FEAT_LDS(128, 256)
#undef HH_FEAT_LDS
    default: return 1;
    }
    int n = (160 * 1024) / lds;
    const int waves = d / 16;
    if (n * waves > 16) n = 16 / waves;  // at most four waves per SIMD
    return n < 1 ? 1 : n;
}

hipError_t launch_feat(int d, int dp, int mode, const FeatParams &p, int grid, hipStream_t st) {
    switch (d * 1000 + dp) {
    case 16016: return launch_feat_d<16, 16>(mode, p, grid, st);
    case 16032: return launch_feat_d<16, 32>(mode, p, grid, st);
    case 32032: return launch_feat_d<32, 32>(mode, p, grid, st);
    case 32064: return launch_feat_d<32, 64>(mode, p, grid, st);
    case 64064: return launch_feat_d<64, 64>(mode, p, grid, st);
    case 64128: return launch_feat_d<64, 128>(mode, p, grid, st);
    case 128128: return launch_feat_d<128, 128>(mode, p, grid, st);
    case 128256: return launch_feat_d<128, 256>(mode, p, grid, st);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_feat_scan(float *S, float *z, int d, int dp, int BH, int nseg, int mode, hipStream_t st) {
    const long perS = (long)feat_padded_dim(dp) * d, perZ = feat_padded_dim(dp);
    const long total = (long)BH * (perS + perZ);
    hipLaunchKernelGGL(feat_scan_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st, S, z, perS, perZ, BH,
                       nseg, mode);
    return hipGetLastError();
}

hipError_t launch_featuremap_variant(int map, int dtype, int d, const void *x, const void *W, const void *b, void *phi,
                                     long BH, int H, int N, hipStream_t st) {
    const long ntok = BH * (long)N;
    if (ntok == 0) return hipSuccess;
    if (dtype == HH_BF16_) {
        const bf16_t *xx = (const bf16_t *)x, *WW = (const bf16_t *)W, *bb = (const bf16_t *)b;
        bf16_t *pp = (bf16_t *)phi;
#define HH_FMV(D)                                                                                      \
    case D:                                                                                            \
        if (map == HH_MAP_EXP_) return launch_fm_variant_d<D, HH_MAP_EXP_>(xx, WW, bb, pp, BH, H, N, st); \
        if (map == HH_MAP_SOFTMAX_) return launch_fm_variant_d<D, HH_MAP_SOFTMAX_>(xx, WW, bb, pp, BH, H, N, st); \
        return launch_fm_variant_d<D, HH_MAP_HEDGEHOG_SOFTMAX_>(xx, WW, bb, pp, BH, H, N, st);
        switch (d) {
            HH_FMV(16) HH_FMV(32) HH_FMV(64) HH_FMV(128)
        default: return hipErrorInvalidValue;
        }
#undef HH_FMV
    }
    hipLaunchKernelGGL(fm_variant_vec_kernel, dim3((unsigned)((ntok + 3) / 4)), dim3(256), 0, st, map, dtype, d, x, W, b,
                       phi, ntok, H, N);
    return hipGetLastError();
}

}  // namespace hh
